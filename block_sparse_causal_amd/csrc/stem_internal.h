// Internal declarations shared by the host library sources.
#ifndef STEM_INTERNAL_H
#define STEM_INTERNAL_H

#include <stdint.h>

// The select kernel keeps one row's candidate keys in registers, at most
// 64 per lane of a 64-wide wavefront.
#define STEM_MAX_SEQ_BLOCKS 4096

#endif
