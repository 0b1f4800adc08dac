// NP-Map of one vector by one wave (Sec. 3.2 of the STILL paper, with the
// Hedgehog form of its Sec. 2):
//   u = P x                       P: [fd/2, d], the learned direction
//   z = ||x|| * u / ||u||         pretrained norm re-injected (z = 0 if u = 0)
//   phi = [softmax(z); softmax(-z)]  (fd values)
// xs: d floats readable by the whole wave (LDS); out: fd floats (LDS), each
// times `scale` (the gate weight of a query; 1 for keys).
#pragma once
#include "device_common.h"

namespace still {

__device__ inline void np_map_wave(const float* xs, const float* __restrict__ P, int d, int fd,
                                   float* out, int lane, float scale = 1.f) {
    float ss = 0.f;
    for (int i = lane; i < d; i += kWave) ss = fmaf(xs[i], xs[i], ss);
    const float nx = sqrtf(wave_sum(ss));
    const int half = fd / 2;
    const bool act = lane < half;
    float u = 0.f;
    if (act) {  // P is 16-byte aligned (the C ABI checks the projections) and d is a multiple of 4
        const float4* pr = reinterpret_cast<const float4*>(P + (size_t)lane * d);
        for (int i = 0; i < d / 4; ++i) {
            const float4 w = pr[i];
            u = fmaf(w.x, xs[4 * i], u);
            u = fmaf(w.y, xs[4 * i + 1], u);
            u = fmaf(w.z, xs[4 * i + 2], u);
            u = fmaf(w.w, xs[4 * i + 3], u);
        }
    }
    const float nu = sqrtf(wave_sum(u * u));
    const float z = nu > 0.f ? nx * (u / nu) : 0.f;
    const float ninf = -__builtin_inff();
    const float m1 = wave_max(act ? z : ninf), m2 = wave_max(act ? -z : ninf);
    const float e1 = act ? expf(z - m1) : 0.f, e2 = act ? expf(-z - m2) : 0.f;
    const float s1 = wave_sum(e1), s2 = wave_sum(e2);
    if (act) {
        out[lane] = scale * (e1 / s1);
        out[half + lane] = scale * (e2 / s2);
    }
}

}  // namespace still
