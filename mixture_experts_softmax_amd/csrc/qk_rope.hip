// QK-Norm + RoPE in one in-place pass, as the NVIDIA Sarvam blog fuses the
// two steps before attention (Table 1, row "QK Norm + RoPE"; the paragraph
// on fused positional embedding): each query and key head is read once,
// RMS-normalised with its learned weight, rotated by its token's position
// and written back.
//
// Lane layout: a lane holds NCH 16-byte chunks of a head that together
// contain whole rotation pairs -- one chunk for the interleaved pairing
// (pairs (2i, 2i+1) inside the chunk), chunk c and chunk c + HD/2 for the
// halves pairing (pairs (i, i + HD/2) across them) -- so the rotation needs
// no lane exchange; LPH = HD / (VEC NCH) lanes per head, 64 / LPH heads side
// by side per round. Wave tasks: a wave takes RPW consecutive rounds of one
// token (all of them for long batches, one for short ones, so that a batch of
// any size has enough waves in flight). A lane's weight chunks (query and
// key) are loaded once; the task's first rounds are loaded before any is
// used (each later round once the round two before it is stored), and while
// they are in flight the wave evaluates its token's rotation table (angle p * theta^(-2i/HD) in float64) into its own LDS
// slice -- no workgroup barrier, a wave's LDS accesses stay in order. The
// head's sum of squares is reduced over its lanes by DPP row moves; each lane
// normalises, rotates and stores.
// HBM-bound: every byte of the q and k heads is read once and written once.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>

#include "common.h"
#include "internal.h"
#include "moe.h"

namespace moe {
namespace {

template <typename E>
struct Elem;
template <>
struct Elem<uint16_t> {  // bf16
  static constexpr int kVec = 8;
  __device__ static float load(uint16_t v) { return bf16_to_f32(v); }
  __device__ static uint16_t store(float v) { return f32_to_bf16(v); }
};
template <>
struct Elem<float> {
  static constexpr int kVec = 4;
  __device__ static float load(float v) { return v; }
  __device__ static float store(float v) { return v; }
};

// cos/sin of pair i at position pos: the frequency theta^(-2i/HD) and the
// angle in float64, reduced to [-pi, pi] in float64, then float32 sincos of
// the reduced angle (absolute error ~1e-7 for any int32 position).
template <int HD>
__device__ inline float2 rope_cs(int i, int pos, double log2_theta) {
  const double inv = exp2(-2.0 * i / HD * log2_theta);
  const double ang = (double)pos * inv;
  const double r = ang - rint(ang * 0.15915494309189535) * 6.283185307179586;
  float sn, cn;
  sincosf((float)r, &sn, &cn);
  return make_float2(cn, sn);
}

constexpr int kQkWavesPerBlock = 4;  // wave tasks per workgroup
// rounds whose loads a task keeps in flight: a round's load is issued once
// the round kQkAhead before it is stored, so a wave's reads and writes
// interleave (all rounds loaded up front measured 3-4% slower at T = 3584)
constexpr int kQkAhead = 2;
// rounds per wave task, at most: 9 chunk loads in flight per lane
__host__ __device__ constexpr int qk_batch(int nch) { return nch == 2 ? 5 : 9; }

// Sum over aligned groups of N lanes (N a power of two): DPP within rows of
// 16 (quad swaps, then the half-row and row mirrors, each pairing lanes of
// the two halves combined so far), shuffles across rows.
template <int N>
__device__ inline float group_sum(float v) {
  auto dpp = [](float x, auto ctrl) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                 decltype(ctrl)::value, 0xF, 0xF,
                                                                 false));
  };
  if constexpr (N >= 2) v += dpp(v, std::integral_constant<int, 0xB1>{});   // quad_perm [1,0,3,2]
  if constexpr (N >= 4) v += dpp(v, std::integral_constant<int, 0x4E>{});   // quad_perm [2,3,0,1]
  if constexpr (N >= 8) v += dpp(v, std::integral_constant<int, 0x141>{});  // row_half_mirror
  if constexpr (N >= 16) v += dpp(v, std::integral_constant<int, 0x140>{}); // row_mirror
  if constexpr (N >= 32) v += __shfl_xor(v, 16, kWave);
  if constexpr (N >= 64) v += __shfl_xor(v, 32, kWave);
  return v;
}

template <typename E, int HD, int STYLE>
__global__ __launch_bounds__(kQkWavesPerBlock * kWave) void qk_norm_rope_kernel(
    E* __restrict__ qkv, const int32_t* __restrict__ positions, const E* __restrict__ qw,
    const E* __restrict__ kw, int T, int n_q, int n_kv, int64_t row_stride, int64_t q_off,
    int64_t k_off, float eps, float theta, int rpw) {
  constexpr int VEC = Elem<E>::kVec;                      // elements per 16-byte chunk
  constexpr int NCH = STYLE == MOE_ROPE_HALVES ? 2 : 1;   // chunks per lane and head
  constexpr int LPH = HD / (VEC * NCH);                   // lanes per head
  constexpr int HPR = kWave / LPH;                        // heads per round
  constexpr int RB = qk_batch(NCH);
  static_assert(LPH <= kWave && kWave % LPH == 0, "a head must sit in one wave");
  __shared__ float2 cs_all[kQkWavesPerBlock][HD / 2];  // (cos, sin) of pair i, per wave

  const int wv = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int nh = n_q + n_kv;
  const int rounds_all = (nh + HPR - 1) / HPR;
  const int wpt = (rounds_all + rpw - 1) / rpw;  // wave tasks per token
  const int task = blockIdx.x * kQkWavesPerBlock + wv;
  const int t = task / wpt;
  if (t >= T) return;  // whole waves: nothing below synchronises across waves
  const int rbeg = (task % wpt) * rpw;
  const int rounds = min(rbeg + rpw, rounds_all);  // this task: rounds [rbeg, rounds)
  float2* cs = cs_all[wv];
  const int l = lane % LPH, hs = lane / LPH;  // lane of the head, head slot of the round
  // element offset of chunk n of this lane within a head
  auto coff = [&](int n) { return (n == 0 ? l : l + HD / (2 * VEC)) * VEC; };
  E* row = qkv + (size_t)t * row_stride;
  auto head_ptr = [&](int h) {  // head h (h < nh)
    return row + (h < n_q ? q_off + (int64_t)h * HD : k_off + (int64_t)(h - n_q) * HD);
  };
  // the lane's weight chunks and the task's head chunks, then the rotation
  // table while they are in flight
  v4i wq[NCH], wk[NCH];
#pragma unroll
  for (int n = 0; n < NCH; ++n) {
    wq[n] = n_q > 0 ? *reinterpret_cast<const v4i*>(qw + coff(n)) : v4i{0, 0, 0, 0};
    wk[n] = n_kv > 0 ? *reinterpret_cast<const v4i*>(kw + coff(n)) : v4i{0, 0, 0, 0};
  }
  v4i xr[RB][NCH];
  auto load_round = [&](int j) {
    const int h = (rbeg + j) * HPR + hs;
    if (rbeg + j < rounds && h < nh) {
#pragma unroll
      for (int n = 0; n < NCH; ++n) xr[j][n] = *reinterpret_cast<const v4i*>(head_ptr(h) + coff(n));
    }
  };
#pragma unroll
  for (int j = 0; j < (RB < kQkAhead ? RB : kQkAhead); ++j) load_round(j);
  {
    const int pos = positions[t];
    const double l2t = log2((double)theta);
#pragma unroll
    for (int i = lane; i < HD / 2; i += kWave) cs[i] = rope_cs<HD>(i, pos, l2t);
  }
  __builtin_amdgcn_wave_barrier();

  const float inv_hd = 1.0f / HD;
#pragma unroll
  for (int j = 0; j < RB; ++j) {
    const int rr = rbeg + j;
    if (rr >= rounds) break;  // uniform across the wave
    const int h = rr * HPR + hs;
    const bool live = h < nh;  // a head slot of the last round may be empty
    float v[NCH][VEC];
    float ss = 0.f;
#pragma unroll
    for (int n = 0; n < NCH; ++n) {
      E xv[VEC];
      *reinterpret_cast<v4i*>(xv) = xr[j][n];
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        v[n][e] = live ? Elem<E>::load(xv[e]) : 0.f;
        ss = fmaf(v[n][e], v[n][e], ss);
      }
    }
    ss = group_sum<LPH>(ss);
    const float rn = 1.0f / sqrtf(ss * inv_hd + eps);
#pragma unroll
    for (int n = 0; n < NCH; ++n) {  // normalised, times the learned weight
      E wv_[VEC];
      *reinterpret_cast<v4i*>(wv_) = (h < n_q) ? wq[n] : wk[n];
#pragma unroll
      for (int e = 0; e < VEC; ++e) v[n][e] = v[n][e] * rn * Elem<E>::load(wv_[e]);
    }

    float o[NCH][VEC];
    if constexpr (STYLE == MOE_ROPE_INTERLEAVED) {
#pragma unroll
      for (int m = 0; m < VEC / 2; ++m) {
        const float2 f = cs[(l * VEC) / 2 + m];
        const float a = v[0][2 * m], b = v[0][2 * m + 1];
        o[0][2 * m] = a * f.x - b * f.y;
        o[0][2 * m + 1] = a * f.y + b * f.x;
      }
    } else {  // pair i = l VEC + e: a in chunk 0, b in chunk 1
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float2 f = cs[l * VEC + e];
        const float a = v[0][e], b = v[1][e];
        o[0][e] = a * f.x - b * f.y;
        o[1][e] = a * f.y + b * f.x;
      }
    }
    if (live) {
#pragma unroll
      for (int n = 0; n < NCH; ++n) {
        E xv[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) xv[e] = Elem<E>::store(o[n][e]);
        *reinterpret_cast<v4i*>(head_ptr(h) + coff(n)) = *reinterpret_cast<const v4i*>(xv);
      }
    }
    if (j + kQkAhead < RB) load_round(j + kQkAhead);
  }
}

template <typename E, int HD>
hipError_t launch_hd(const moe_qk_shape_t& s, void* qkv, const int32_t* pos, const void* qw,
                     const void* kw, hipStream_t st) {
  const auto* q = static_cast<const E*>(qw);
  const auto* k = static_cast<const E*>(kw);
  // rounds per wave task: enough tasks to keep the chip's waves busy (a
  // short batch splits each token over several waves), at most qk_batch
  const int nch = s.style == MOE_ROPE_HALVES ? 2 : 1;
  const int hpr = kWave / (HD / (Elem<E>::kVec * nch));
  const int rounds = (s.n_q + s.n_kv + hpr - 1) / hpr;
  const long long target = 2048;  // wave tasks
  const int rpw = (int)std::max(1LL, std::min<long long>(
                                         std::min(rounds, qk_batch(nch)),
                                         (long long)s.T * rounds / target));
  const long long tasks = (long long)s.T * ((rounds + rpw - 1) / rpw);
  const dim3 grid((unsigned)((tasks + kQkWavesPerBlock - 1) / kQkWavesPerBlock));
  const dim3 block(kQkWavesPerBlock * kWave);
  if (s.style == MOE_ROPE_INTERLEAVED)
    hipLaunchKernelGGL((qk_norm_rope_kernel<E, HD, MOE_ROPE_INTERLEAVED>), grid, block, 0, st,
                       static_cast<E*>(qkv), pos, q, k, s.T, s.n_q, s.n_kv, s.row_stride,
                       s.q_offset, s.k_offset, s.eps, s.theta, rpw);
  else
    hipLaunchKernelGGL((qk_norm_rope_kernel<E, HD, MOE_ROPE_HALVES>), grid, block, 0, st,
                       static_cast<E*>(qkv), pos, q, k, s.T, s.n_q, s.n_kv, s.row_stride,
                       s.q_offset, s.k_offset, s.eps, s.theta, rpw);
  return hipGetLastError();
}

template <typename E>
hipError_t launch_e(const moe_qk_shape_t& s, void* qkv, const int32_t* pos, const void* qw,
                    const void* kw, hipStream_t st) {
  switch (s.head_dim) {
    case 64: return launch_hd<E, 64>(s, qkv, pos, qw, kw, st);
    case 128: return launch_hd<E, 128>(s, qkv, pos, qw, kw, st);
    case 256: return launch_hd<E, 256>(s, qkv, pos, qw, kw, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_qk_norm_rope(const moe_qk_shape_t& s, void* qkv, const int32_t* positions,
                               const void* q_weight, const void* k_weight, hipStream_t st) {
  if (s.dtype == MOE_DTYPE_BF16)
    return launch_e<uint16_t>(s, qkv, positions, q_weight, k_weight, st);
  return launch_e<float>(s, qkv, positions, q_weight, k_weight, st);
}

}  // namespace moe
