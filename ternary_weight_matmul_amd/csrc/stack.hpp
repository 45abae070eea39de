// The whole-stack decode step (k_stack.hip): its arguments and launcher
// (internal to the library).
#pragma once
#include "launch.hpp"

namespace mmf {

// One block of the stack as the kernel reads it (a table in device memory,
// written by mmf_stack_decode_bind). w / mu / gain in the order i, f, g, o,
// gate, down; h is the block's recurrent state [b][d] fp32, updated in place.
struct StackLayer {
    const uint32_t *w[6];
    const float *mu[6];
    const float *gain[6];
    const float *g_norm_w;
    float *h;
    float eps;
    int32_t pad;
};

constexpr int kStackBarWords = 19 * 64;  // barrier words (a 256-byte line each)

struct StackArgs {
    const StackLayer *layers;  // [n_layers], device memory
    int n_layers, d, inner, b;
    ActType act_type;
    const void *x;             // [b][d], activation dtype
    void *out;                 // [b][d], activation dtype
    void *act[2];              // block outputs between blocks, [b][d] activation dtype
    float *g, *x1, *z;         // [b][d], [b][d], [b][inner] fp32
    int8_t *codes;             // [16][max(d, inner)]
    float *s;                  // [16]
    int32_t *sumq;             // [16]
    unsigned *bar;             // kStackBarWords, zeroed by the launcher before each launch
};

// Why the shape cannot run (nullptr if it can): b in 1..16, d and inner
// multiples of 256, and the codes of 16 rows fit in LDS.
const char *stack_decode_unsupported(int64_t b, int d, int inner);
hipError_t launch_stack_decode(const StackArgs &a, hipStream_t st, std::string *path);
// Barrier waits that expired in any launch since the library was loaded (synchronous).
hipError_t stack_decode_expired_waits(unsigned *count);

}  // namespace mmf
