// Helpers shared by the row kernels (LayerNorm / RMSNorm forward and
// backward): the 256-thread team that owns one row at a time, its weights
// and its fixed-order row sums.
#pragma once

#include "nh_internal.hpp"

namespace nh {

constexpr int kTeam = 256;
constexpr int kTeamWaves = kTeam / kWave;
constexpr int kMaxTeams = 4;
constexpr int kRedFloats = 2 * kMaxTeams * kTeamWaves * 2;  // double-buffered row sums

__device__ __forceinline__ float load_param(const void *w, int w_bf16, int col)
{
    return w_bf16 ? to_f32(static_cast<const uint16_t *>(w)[col]) : static_cast<const float *>(w)[col];
}

// The weight group of a thread, widened to fp32 once per kernel (NULL: 1.0).
template <int VEC>
struct WeightGroup {
    float v[VEC];
    __device__ __forceinline__ void load(const void *w, int w_bf16, int col)
    {
        if (w == nullptr) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) v[e] = 1.f;
        } else if (w_bf16) {
            load_vec<uint16_t, VEC>(static_cast<const uint16_t *>(w) + col, v);
        } else {
            load_vec<float, VEC>(static_cast<const float *>(w) + col, v);
        }
    }
    __device__ __forceinline__ float get(int e) const { return v[e]; }
};

// Fixed-order sum of the 4 wave results of a team for two quantities.
__device__ __forceinline__ void team_sum2(float *red, int team, int wave, int lane,
                                          float &a, float &b)
{
    a = wave_sum(a);
    b = wave_sum(b);
    if (lane == 0) {
        red[(team * kTeamWaves + wave) * 2 + 0] = a;
        red[(team * kTeamWaves + wave) * 2 + 1] = b;
    }
    lds_barrier();
    float sa = red[(team * kTeamWaves) * 2 + 0];
    float sb = red[(team * kTeamWaves) * 2 + 1];
#pragma unroll
    for (int w = 1; w < kTeamWaves; ++w) {
        sa += red[(team * kTeamWaves + w) * 2 + 0];
        sb += red[(team * kTeamWaves + w) * 2 + 1];
    }
    a = sa;
    b = sb;
}

} // namespace nh
