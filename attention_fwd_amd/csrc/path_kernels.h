// path_kernels.h -- launch interface between the C ABI and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace path {

struct PrepArgs {
    const void *q, *k, *v, *w;
    const float *beta, *logf;
    void *out;
    float *lse;
    void *ws;
    int B, H, L, d;
    float scale;
    // Producer of w and beta fused into the prep (when conv_w is set): w then
    // points at the pre-convolution rows [B, H, L, d], conv_w at the causal
    // width-3 depthwise weights [H, d, 3] and zbeta at the pre-sigmoid values
    // [B, H, L] (beta is unused); beta = 2 sigmoid(z), capped at beta_clip > 0.
    const float *conv_w, *zbeta;
    float beta_clip;
};

struct FwdArgs {
    void *out;
    float *lse;
    const void *ws;
    int B, H, L, d;
    float scale;
    int fox;
    int skip;  // with fox: skip key blocks whose contribution is provably below 2^-kSkipLog2
};

struct DecodeArgs {
    void *kc, *vc;
    int64_t n, ncap;
    const void *q, *w;
    const float *beta;
    const float *logf;  // forget gate: log f_t [B, H], or NULL
    float *fcache;      // forget gate: c_j = sum_{s<=j} log f_s per cached row [B, H, ncap], or NULL
    const void *knew, *vnew;
    void *out;
    float *lse;
    void *ws;
    int B, H, d;
    float scale;
    int nsplit;
    int64_t chunk;
};

// The producer of w and beta for one decode step (path_decode_produce_kernel).
struct ProduceArgs {
    const void *wraw;      // [B, H, d] element type: the current token's raw row x_t
    const float *conv_w;   // [H, d, 3]
    const float *zbeta;    // [B, H]
    float beta_clip;       // 0: no cap
    void *state;           // [B, H, 2, d] element type: x_{t-2}, x_{t-1}; moved on to x_{t-1}, x_t
    void *w_out;           // [B, H, d] element type: y_t rounded
    float *beta_out;       // [B, H]: beta_t / max(||y_t||^2, 1e-24)
    int B, H, d;
};

struct CacheArgs {
    const void *ws, *v;
    const float *logf;  // prefix log-forget gate [B, H, L] or NULL
    float *fcache;      // its inclusive prefix sums [B, H, ncap] or NULL
    void *kc, *vc;
    int64_t ncap;
    int B, H, L, d;
};

hipError_t launch_prep(const PrepArgs &a, bool bf16, hipStream_t st);
hipError_t launch_fwd(const FwdArgs &a, bool bf16, hipStream_t st);
hipError_t launch_decode(const DecodeArgs &a, bool bf16, hipStream_t st);
hipError_t launch_decode_produce(const ProduceArgs &a, bool bf16, hipStream_t st);
hipError_t launch_cache(const CacheArgs &a, bool bf16, hipStream_t st);

// Rows one decode workgroup covers per iteration (bf16, d = 64: 32 lane groups x
// 8 rows; the other element types and head sizes cover a divisor of it).
constexpr int kDecodeRowStep = 256;

// Decode split plan: rows per split and number of splits for n attending rows.
void decode_plan(int64_t BH, int64_t rows, int *nsplit, int64_t *chunk);

// The decode kernels' fixed scratch array (for callers that cannot allocate):
// its size in bytes, and its address on the current device (looked up once per
// device, then cached).
size_t decode_scratch_bytes();
hipError_t decode_scratch(void **ptr);

}  // namespace path
