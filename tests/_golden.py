"""Reader of the small text fixtures under tests/golden/ (each value there
carries the citation of the page that prints it)."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def pages_parameters() -> dict:
    out = {}
    with open(os.path.join(GOLDEN, "pages_parameters.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                name, value = line.split()
                out[name] = float(value)
    return out
