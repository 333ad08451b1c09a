// Weight-stream probe: the read pattern of the tall-tile gate/up kernel with
// nothing else. ntiles tiles of 1 MiB (256 rows of 4096 bytes), one per
// workgroup, each read in 32 K steps of 256 rows x 128 bytes, every 16-byte
// piece of a step by one lane (8 rows of 128 bytes per wave load, chunks
// swizzled by row as in the kernel). Three ways to keep steps in flight:
//   MODE 0  direct-to-LDS loads (global_load_lds_dwordx4) into D + 1 stages
//           of 32 KiB; before issuing step kt + D a wave waits for its step kt
//   MODE 1  register loads that the compiler schedules freely (the values are
//           folded into a checksum, so no load is dropped)
//   MODE 2  register loads D steps ahead, each step written to one of two LDS
//           stages when it is due (an empty asm with a memory clobber keeps
//           the stores and the issue order)
// The workgroup's LDS is dynamic, so the caller also sets how many
// workgroups share a CU. Test infrastructure: not part of libmoe.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt out of range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
template <class Fn, int... Ks>
__device__ inline void each_impl(Fn&& f, std::integer_sequence<int, Ks...>) {
  (f(std::integral_constant<int, Ks>{}), ...);
}
template <int N, class Fn>
__device__ inline void each(Fn&& f) {
  each_impl(f, std::make_integer_sequence<int, N>{});
}

constexpr int kSteps = 32, kRowBytes = 4096, kTileBytes = 256 * kRowBytes, kStage = 32768;

template <int NW, int D, int MODE>
__global__ __launch_bounds__(NW * 64) void stream_probe_kernel(const uint8_t* __restrict__ w,
                                                               int ntiles, int* __restrict__ sink) {
  constexpr int NP = 2048 / (NW * 64);  // 16-byte pieces per thread per step
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  if ((int)blockIdx.x >= ntiles) return;
  const uint8_t* base = w + (size_t)blockIdx.x * kTileBytes;
  const uint8_t* src[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int r = 8 * (NP * wave + i) + (lane >> 3);  // < 256
    src[i] = base + (size_t)r * kRowBytes + ((lane & 7) ^ (r & 7)) * 16;
  }
  if constexpr (MODE == 0) {
    auto issue = [&](int kt) {
      uint8_t* st = lds + (kt % (D + 1)) * kStage;
#pragma unroll
      for (int i = 0; i < NP; ++i)
        __builtin_amdgcn_global_load_lds((const void*)(src[i] + kt * 128),
                                         (lds_void_t*)(st + (NP * wave + i) * 1024), 16, 0, 0);
    };
#pragma unroll
    for (int s = 0; s < D; ++s) issue(s);
    each<kSteps>([&](auto kc) {
      constexpr int kt = decltype(kc)::value;
      constexpr int later = (kSteps - 1 - kt) < (D - 1) ? (kSteps - 1 - kt) : (D - 1);
      wait_vmcnt<later * NP>();  // step kt landed
      if constexpr (kt + D < kSteps) issue(kt + D);
    });
  } else if constexpr (MODE == 1) {
    v4i r[D][NP];
    v4i sum = {0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < D; ++s)
#pragma unroll
      for (int i = 0; i < NP; ++i) r[s][i] = *reinterpret_cast<const v4i*>(src[i] + s * 128);
    each<kSteps>([&](auto kc) {
      constexpr int kt = decltype(kc)::value;
#pragma unroll
      for (int i = 0; i < NP; ++i) sum ^= r[kt % D][i];
      if constexpr (kt + D < kSteps) {
#pragma unroll
        for (int i = 0; i < NP; ++i)
          r[kt % D][i] = *reinterpret_cast<const v4i*>(src[i] + (kt + D) * 128);
      }
    });
    if ((sum.x ^ sum.y ^ sum.z ^ sum.w) == 0x7fffffff) sink[0] = 1;
  } else {
    v4i r[D][NP];
#pragma unroll
    for (int s = 0; s < D; ++s)
#pragma unroll
      for (int i = 0; i < NP; ++i) r[s][i] = *reinterpret_cast<const v4i*>(src[i] + s * 128);
    each<kSteps>([&](auto kc) {
      constexpr int kt = decltype(kc)::value;
      uint8_t* st = lds + (kt & 1) * kStage;
#pragma unroll
      for (int i = 0; i < NP; ++i)
        *reinterpret_cast<v4i*>(st + (NP * wave + i) * 1024 + lane * 16) = r[kt % D][i];
      asm volatile("" ::: "memory");
      if constexpr (kt + D < kSteps) {
#pragma unroll
        for (int i = 0; i < NP; ++i)
          r[kt % D][i] = *reinterpret_cast<const v4i*>(src[i] + (kt + D) * 128);
      }
    });
  }
}

template <int NW, int D, int MODE>
int launch(const uint8_t* w, int ntiles, int* sink, int lds_bytes, hipStream_t s) {
  const int need = MODE == 0 ? (D + 1) * kStage : MODE == 2 ? 2 * kStage : 0;
  if (lds_bytes < need || lds_bytes > 163840) return -2;
  auto k = stream_probe_kernel<NW, D, MODE>;
  if (hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes) !=
      hipSuccess)
    return -3;
  hipLaunchKernelGGL(k, dim3(ntiles), dim3(NW * 64), lds_bytes, s, w, ntiles, sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // namespace

// config: 0 dma 8 waves 2 ahead, 1 dma 8w 3 ahead, 2 dma 16w 2 ahead,
// 3 reg 8w, 4 reg 16w, 5 reg->lds 8w 2 ahead, 6 reg->lds 8w 3 ahead,
// 7 reg->lds 16w 2 ahead. w holds ntiles MiB. Returns 0 or a negative code.
extern "C" int stream_probe(int config, const void* w, int ntiles, int* sink, int lds_bytes,
                            void* stream) {
  const uint8_t* p = static_cast<const uint8_t*>(w);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (ntiles <= 0 || w == nullptr || sink == nullptr) return -1;
  switch (config) {
    case 0: return launch<8, 2, 0>(p, ntiles, sink, lds_bytes, s);
    case 1: return launch<8, 3, 0>(p, ntiles, sink, lds_bytes, s);
    case 2: return launch<16, 2, 0>(p, ntiles, sink, lds_bytes, s);
    case 3: return launch<8, 2, 1>(p, ntiles, sink, lds_bytes, s);
    case 4: return launch<16, 2, 1>(p, ntiles, sink, lds_bytes, s);
    case 5: return launch<8, 2, 2>(p, ntiles, sink, lds_bytes, s);
    case 6: return launch<8, 3, 2>(p, ntiles, sink, lds_bytes, s);
    case 7: return launch<16, 2, 2>(p, ntiles, sink, lds_bytes, s);
  }
  return -1;
}
