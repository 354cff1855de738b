// api_internal.h -- descriptor checks shared by the host-side C ABI files of
// libgdntree (not installed, not part of the ABI, not exported).
#pragma once

#include "gdn_tree.h"
#include "gdn_tree_attn.h"

namespace gdn {

// The synchronous checks every entry point of gdn_tree.h / gdn_tree_attn.h
// makes on its descriptor before anything is enqueued.
__attribute__((visibility("hidden"))) gdn_status check_tree_desc(const gdn_tree_desc* d);
__attribute__((visibility("hidden"))) gdn_status check_attn_desc(const gdn_attn_desc* d);

}  // namespace gdn
