// Hooks of api.cpp for entry points implemented in other source files of the
// library.  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/saf3r.h"

// One layer exactly as saf_sparse_attention computes it, on the caller's
// stream only (no side stream, no stream or event creation, no per-launch
// timing), with the workspace ws of ws_bytes.  *ws_need receives the bytes
// the plan needs; a plan needing more than ws_cap fails with
// SAF_EUNSUPPORTED.  ws = NULL only validates the plan and reports *ws_need.
saf_status_t saf_layer_internal(saf_ctx_t *c, const saf_head_plan_t *plan, const void *q, const void *k,
                                const void *v, void *o, saf_layout_t lay, const int32_t *vert_idx, int64_t vert_ld,
                                void *ws, size_t ws_bytes, void *stream, size_t ws_cap, size_t *ws_need);

// Record an error message on the context and return the status.
saf_status_t saf_fail_internal(saf_ctx_t *c, int32_t status, const char *msg);
