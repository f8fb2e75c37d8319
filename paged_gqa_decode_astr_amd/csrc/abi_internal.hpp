// Host-side helpers shared by the C ABI sources (api.cpp, graph.cpp).
#pragma once

#include <stddef.h>

#include "astr_attn.h"

namespace astr {

// Records a printf-style message for astr_last_error() and returns `status`.
int fail(int status, const char* fmt, ...);
// Clears the message and returns ASTR_OK.
int ok();
const char* last_error();

// Validates and enqueues one decode call (with the fused append when nkv is
// not null): the body of astr_paged_decode / astr_paged_decode_append.
// With use_scratch, workspace and workspace_bytes are ignored and the
// partials go to the library's scratch array (astr_paged_decode_noalloc).
int decode_impl(const astr_paged_args* a, const astr_new_kv* nkv, void* workspace, size_t workspace_bytes,
                void* stream, bool use_scratch = false);

}  // namespace astr
