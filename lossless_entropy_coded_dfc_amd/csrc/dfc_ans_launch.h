// dfc_ans_launch.h - launcher of the interleaved rANS decoder, called by the
// batched decode entry points (internal to libdfc).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "dfc.h"

namespace dfc {

// Layout-specific checks of one ANS batch item (the common ones are done).
dfc_status ans_check_item(const dfc_batch_item &it);
// One launch decoding the ANS items items[idx[0..count)].
dfc_status ans_launch(const dfc_batch_item *items, const uint32_t *idx, uint32_t count, uint32_t *status,
                      hipStream_t stream);
// One workgroup of `threads` threads derives the slot table of an ANS
// container the way the decoder does and writes it to dst (16 KB).
dfc_status ans_derive_tables(const void *blob_dev, const dfc_info &info, uint32_t threads, void *dst,
                             hipStream_t stream);

}  // namespace dfc
