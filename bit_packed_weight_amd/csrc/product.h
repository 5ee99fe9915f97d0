// Product entry shared by the C-ABI calls (api.cpp) and the fixed-scratch
// entry point (scratch.hip): validation, workspace sizing and dispatch.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/bpw.h"

namespace bpw {

// Validate a weight descriptor (formats, sizes, alignment); BPW_OK or a status
// with the thread's error text set.
int check_weights(const bpw_weights* w);
// Validate the product arguments (weights, activations, scales, output) on
// the host, without looking at a workspace or the device.
int check_product_args(const bpw_weights* w, const void* x, int x_dtype, const float* x_scale, int64_t m,
                       void* y, int y_dtype);
// The current device is the stream's device (when the stream is not NULL) and
// a gfx950 (checked once per device).
int check_current_device(void* stream);
// Device workspace bytes a product needs for (weights, M, activation type,
// entry), rounded up to 256; the descriptor must already be valid.
size_t workspace_need(const bpw_weights* w, int64_t m, int x_dtype, int entry);
// Validate every argument, then launch the product on `stream` with `ws`
// (ws_bytes long) as its workspace.
int run_product(bool gemv, const bpw_weights* w, const void* x, int x_dtype, const float* x_scale,
                int64_t m, void* y, int y_dtype, void* ws, size_t ws_bytes, void* stream);

}  // namespace bpw
