// Internal launch interface between the C ABI layer (api.cpp) and the
// kernel translation units.  Every launcher assumes validated arguments and
// returns the hipError_t of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace w4a4 {

// ---- activation path (transform_quant.hip) --------------------------------
enum class TqPath { Fused, Cols, Split };

// Activation quantizer of one call.  Dynamic (steps == nullptr): per-token
// scale alpha * max|z| / 7.  Static: steps fixed offline, either one step for
// the whole tensor (the token scale is that step) or one step per channel
// (codes round z_k / step_k; the token scale written is 1).
struct ActQuant {
    float alpha;
    const float* steps;
    bool per_channel;
};

TqPath tq_select_path(int M, int n1, int n2, bool has_c);
size_t tq_workspace_bytes(int M, int n1, int n2, bool has_c);

// quantize=true: Xq/s_x outputs; quantize=false: Z (fp32 [M,K]) output.
hipError_t tq_launch(const uint16_t* X, int M, int n1, int n2, const float* P1,
                     const float* P2, const float* c, ActQuant aq, bool quantize,
                     uint8_t* Xq, float* s_x, float* Z, void* ws, size_t ws_bytes,
                     hipStream_t stream);

// ---- GEMM (gemm.hip) -------------------------------------------------------
struct GemmArgs {
    const uint8_t* Xq;
    const float* s_x;
    const uint8_t* Wq;
    const uint16_t* s_w;
    const uint16_t* z_w;
    uint16_t* Y;     // fp16 output (mode fp16)
    int32_t* D;      // int32 output (mode i32)
    int M, N, K, group_size;
    bool asym;
};

size_t gemm_workspace_bytes(int M, int N, int K, int group_size);
// name of the configuration gemm_launch would use (launches nothing)
const char* gemm_kernel_name(const GemmArgs& a, bool i32_out);
hipError_t gemm_launch(const GemmArgs& a, bool i32_out, void* ws, size_t ws_bytes,
                       hipStream_t stream);

// ---- single-kernel decode layer (linear_decode.hip) --------------------------
size_t linear_decode_workspace_bytes(int M, int n1, int n2);
// 0: supported; 1: shape not covered; 2: too much LDS; 3: the producers
// exceed the device's resident capacity
int linear_decode_check(int M, int n1, int n2, int N, int K, int group_size, bool asym,
                        int* cap);
hipError_t linear_decode_launch(const uint16_t* X, int M, int n1, int n2, const float* P1,
                                const float* P2, ActQuant aq, const GemmArgs& g, void* ws,
                                uint32_t* sync, hipStream_t stream);

// ---- offline weight preparation (weights.hip) ------------------------------
size_t merge_workspace_bytes(int n1, int n2, int K);
// returns hipSuccess and sets *singular when a factor has no usable pivot
hipError_t merge_launch(const float* W, int N, int K, int n1, int n2, const float* P1,
                        const float* P2, const float* c, float* Wt, void* ws,
                        hipStream_t stream, bool* singular);
// Wm[n, k] = Wt[n, k] * steps[k] (fp32, one rounding); Wm may equal Wt
hipError_t migrate_steps_launch(const float* Wt, int N, int K, const float* steps, float* Wm,
                                hipStream_t stream);
hipError_t pack_weights_launch(const float* Wt, int N, int K, int group_size, bool asym,
                               float alpha_w, uint8_t* Wq, uint16_t* s_w, uint16_t* z_w,
                               hipStream_t stream);

}  // namespace w4a4
