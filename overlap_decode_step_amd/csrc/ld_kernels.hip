// ld_kernels.hip - kernels of the decode step for gfx950 and their launch
// wrappers (the host runtime calls only the wrappers in ld_launch.h).
//
//  k_qkv / k_attn / k_o / k_gu / k_d / k_lm : one kernel per stage, used by
//      the whole-kernel-wait and tile-flag modes;
//  k_mega : one persistent kernel per step whose workgroups run every stage
//      of every layer in order, synchronising on the same readiness counters
//      (the single-kernel decode of Hazy Research, "Look Ma, No Bubbles!
//      Designing a Low-Latency Megakernel for Llama-1B");
//  k_gen_normal / k_fill16 / k_gen_kv : seeded synthetic inputs.
// All decode kernels use dynamic LDS: a scratch area, then the staged input
// vectors or the attention tiles.
#include <mutex>

#include "ld_launch.h"
#include "ld_stages.hpp"
#include "../../synth/ld_synth.h"

namespace ld {

// 512-thread workgroups.  The persistent kernel runs one per CU, so each wave
// may hold up to 256 VGPRs (the weight-block rings of the GEMV engine live in
// registers); the stage kernels are held to 128 (four waves per SIMD) so that
// two of them fit on a CU side by side in the tile-flag mode.
constexpr int kMaxThreads = kBlockThreads;
constexpr int kStageWavesPerSimd = 4;
// At 64 rows the whole-kernel-wait and graph modes (one kernel on a CU at a
// time) run stage kernels built for two waves per SIMD, so that the MFMA
// engine takes the batch in one 64-row pass like the persistent kernel
// (measured 5.63 -> 5.03 ms per step at batch 64; at batch 16 the deeper
// weight ring of these builds was 9% slower, so 16 and 32 rows keep the
// four-wave builds, as does the tile-flag mode).
constexpr int kStageWavesFull = 2;
constexpr int kFullNb = 64;
template <int WPS>
constexpr int kStageRing = WPS == kStageWavesFull ? kMfmaRingBig : kMfmaRingSmall;

template <int NB, int WPS = kStageWavesPerSimd>
__global__ __launch_bounds__(kMaxThreads, WPS) void k_qkv(Params P, int l) {
  extern __shared__ __align__(16) char smem[];
  stage_qkv<NB, kStageRing<WPS>>(P, l, blockIdx.x, gridDim.x, smem);
}

__global__ __launch_bounds__(kMaxThreads, kStageWavesPerSimd) void k_attn(Params P, int l) {
  extern __shared__ __align__(16) char smem[];
  scratch_init(smem);
  stage_attn<true>(P, l, blockIdx.x, gridDim.x, smem, [] {});
}

template <int NB, int WPS = kStageWavesPerSimd>
__global__ __launch_bounds__(kMaxThreads, WPS) void k_o(Params P, int l) {
  extern __shared__ __align__(16) char smem[];
  stage_o<NB, kStageRing<WPS>>(P, l, blockIdx.x, gridDim.x, smem);
}

template <int NB, int WPS = kStageWavesPerSimd>
__global__ __launch_bounds__(kMaxThreads, WPS) void k_gu(Params P, int l) {
  extern __shared__ __align__(16) char smem[];
  GuBlock ring[kPfGu];
  stage_gu<NB, kStageRing<WPS>>(P, l, blockIdx.x, gridDim.x, smem, ring, false);
}

template <int NB, int WPS = kStageWavesPerSimd>
__global__ __launch_bounds__(kMaxThreads, WPS) void k_d(Params P, int l) {
  extern __shared__ __align__(16) char smem[];
  stage_d<NB, kStageRing<WPS>>(P, l, blockIdx.x, gridDim.x, smem);
}

template <int NB, int WPS = kStageWavesPerSimd>
__global__ __launch_bounds__(kMaxThreads, WPS) void k_lm(Params P, int l) {
  extern __shared__ __align__(16) char smem[];
  stage_lm<NB, kStageRing<WPS>>(P, blockIdx.x, gridDim.x, smem);
}

// unfused-MLP ablation: the projection GEMVs and the elementwise kernels
// (the same builds per batch size as the fused stage's kernel they replace)
template <int NB, int WPS = kStageWavesPerSimd>
__global__ __launch_bounds__(kMaxThreads, WPS) void k_mlp_proj(Params P, int l, int which) {
  extern __shared__ __align__(16) char smem[];
  stage_mlp_proj<NB, kStageRing<WPS>>(P, l, which, blockIdx.x, gridDim.x, smem);
}

__global__ void k_mlp_elem(Params P, int op, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    mlp_elementwise(P, op, i);
}

// The persistent kernel reads its argument block for every stage straight
// from the kernel-argument segment (invariant constant memory), so the
// compiler reloads fields with scalar loads where a stage uses them.  (Kept in
// one value across the layer loop, the ~100 dwords of fields did not fit the
// scalar registers and were spilled to vector-register lanes: some 2000 lane
// reads in the loop body.  Forcing a reload of every field at each stage
// start was measured slower than letting the compiler choose.)
__device__ __forceinline__ Params fresh_params() {
#if defined(__HIP_DEVICE_COMPILE__)
  using ConstParams = const __attribute__((address_space(4))) Params;
  return *(ConstParams*)__builtin_amdgcn_kernarg_segment_ptr();
#else
  return Params{};  // host pass: never called
#endif
}

template <int NB>
__global__ __launch_bounds__(kMaxThreads) void k_mega(Params P0) {
  extern __shared__ __align__(16) char smem[];
  scratch_init(smem);
  const int wg = blockIdx.x, nwg = gridDim.x;
  const int L = P0.D.L;
#pragma clang loop unroll(disable)
  for (int l = 0; l < L; ++l) {
    stage_qkv<NB, kMfmaRingBig>(fresh_params(), l, wg, nwg, smem);
    // workgroups without an attention item load their first SwiGLU weight
    // blocks while attention runs, into registers and LDS (VALU engine)
    GuBlock gring[kPfGu];
    bool gpre = false;
    int gnl = 0;
    {
      const Params P = fresh_params();
      stage_attn<false>(P, l, wg, nwg, smem, [&] {
        if constexpr (NB < kMfmaMinBatch) {
          gnl = gu_prefetch<NB>(P, l, wg, nwg, gring, smem);
          gpre = true;
        }
      });
    }
    __syncthreads();
    stage_o<NB, kMfmaRingBig>(fresh_params(), l, wg, nwg, smem);
    stage_gu<NB, kMfmaRingBig>(fresh_params(), l, wg, nwg, smem, gring, gpre, gnl);
    stage_d<NB, kMfmaRingBig>(fresh_params(), l, wg, nwg, smem);
  }
  stage_lm<NB, kMfmaRingBig>(fresh_params(), wg, nwg, smem);
}

// ---------------------------------------------------------- generators

__global__ void k_gen_normal(uint16_t* dst, int64_t n, uint64_t key, uint64_t index0,
                             float kappa) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    dst[i] = ls_normal_bf16(key, index0 + (uint64_t)i, kappa);
}

__global__ void k_fill16(uint16_t* dst, int64_t n, uint16_t v) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = v;
}

// Debug poison: blockIdx.y < r.count fills range blockIdx.y with fp32 quiet
// NaNs; blockIdx.y == r.count fills the appended cache rows with bf16 quiet
// NaNs (a position outside [0, max_seq) is skipped: the step reports it).
__global__ void k_poison(PoisonRanges r, uint16_t* kc, uint16_t* vc, const int32_t* pos, int rows,
                         int M, int L, int max_batch, int nkv, int max_seq, int d) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if ((int)blockIdx.y < r.count) {
    uint32_t* p = r.p[blockIdx.y];
    for (int64_t i = i0; i < r.n[blockIdx.y]; i += stride) p[i] = 0x7FC00000u;
    return;
  }
  // (row, layer, kv head, channel)
  const int64_t n = (int64_t)rows * L * nkv * d;
  for (int64_t e = i0; e < n; e += stride) {
    const int c = (int)(e % d);
    int64_t q = e / d;
    const int h = (int)(q % nkv);
    q /= nkv;
    const int l = (int)(q % L);
    const int b = (int)(q / L);
    const int p = pos[b];
    if ((unsigned)p >= (unsigned)max_seq) continue;
    const int64_t off = ((((int64_t)l * max_batch + b / M) * nkv + h) * max_seq + p) * d + c;
    kc[off] = 0x7FC0u;
    vc[off] = 0x7FC0u;
  }
}

// KV prefill of one layer: blockIdx.y = seq * n_kv + head; positions < len[seq].
__global__ void k_gen_kv(uint16_t* kc, uint16_t* vc, const int* len, int n_kv, int max_seq,
                         int d, uint64_t kkey, uint64_t vkey, float kappa) {
  const int bh = blockIdx.y, b = bh / n_kv, h = bh - b * n_kv;
  const int64_t n = (int64_t)len[b] * d;
  const int64_t base = (int64_t)bh * max_seq * d;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += stride) {
    const uint64_t pos = (uint64_t)(e / d), i = (uint64_t)(e % d);
    const uint64_t idx = ls_kv_index((uint64_t)b, (uint64_t)n_kv, (uint64_t)h, pos, (uint64_t)d, i);
    kc[base + e] = ls_normal_bf16(kkey, idx, kappa);
    vc[base + e] = ls_normal_bf16(vkey, idx, kappa);
  }
}

// ------------------------------------------------ allocation-free KV fill
//
// The KV fill reads the prefill lengths from device memory.  ld_fill_kv
// copies them into a buffer from hipMalloc; its allocation-free variant keeps
// them in this file-scope device array instead (every GPU the library runs on
// holds its own copy until the process ends).  Host code reaches the array
// only through the address hipGetSymbolAddress returns for the current
// device; its name is not a device address in host code.  Every call on a
// device shares that device's copy, so such calls that overlap on one device
// (on different streams) race.
constexpr int kScratchLens = 64;  // lengths at most (max_batch <= 64)
static __device__ __align__(256) int32_t scratch[kScratchLens];

struct ScratchLens {
  int32_t v[kScratchLens];
};

// Writes the call's n lengths (passed by value) and zeros after them.
__global__ void k_put_lens(int32_t* dst, ScratchLens lens, int n) {
  const int i = threadIdx.x;
  if (i < kScratchLens) dst[i] = i < n ? lens.v[i] : 0;
}

constexpr int kMaxScratchDevices = 64;
static std::mutex g_scratch_mu;
static int32_t* g_scratch[kMaxScratchDevices] = {};

hipError_t scratch_lens_ptr(int32_t** out, int* capacity) {
  *out = nullptr;
  *capacity = kScratchLens;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[dev] = static_cast<int32_t*>(p);
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

hipError_t launch_put_lens(int32_t* dst, const int32_t* host_lens, int n, hipStream_t s) {
  if (n < 0 || n > kScratchLens) return hipErrorInvalidValue;
  ScratchLens lens{};
  for (int i = 0; i < n; ++i) lens.v[i] = host_lens[i];
  hipLaunchKernelGGL(k_put_lens, dim3(1), dim3(kScratchLens), 0, s, dst, lens, n);
  return hipGetLastError();
}

// ------------------------------------------------------------ wrappers

template <int NB, int WPS = kStageWavesPerSimd>
static const void* stage_fn(int stage) {
  switch (stage) {
    case 0: return reinterpret_cast<const void*>(&k_mega<NB>);
    case kSQkv: return reinterpret_cast<const void*>(&k_qkv<NB, WPS>);
    case kSAttn: return reinterpret_cast<const void*>(&k_attn);
    case kSO: return reinterpret_cast<const void*>(&k_o<NB, WPS>);
    case kSGu: return reinterpret_cast<const void*>(&k_gu<NB, WPS>);
    case kSD: return reinterpret_cast<const void*>(&k_d<NB, WPS>);
    case kSLm: return reinterpret_cast<const void*>(&k_lm<NB, WPS>);
    case kSMlpProj: return reinterpret_cast<const void*>(&k_mlp_proj<NB, WPS>);
    default: return nullptr;
  }
}

static const void* kernel_ptr(int stage, int nb, bool full = false) {
  if (full && nb == kFullNb) return stage_fn<kFullNb, kStageWavesFull>(stage);
  switch (nb) {
    case 1: return stage_fn<1>(stage);
    case 2: return stage_fn<2>(stage);
    case 4: return stage_fn<4>(stage);
    case 8: return stage_fn<8>(stage);
    case 16: return stage_fn<16>(stage);
    case 32: return stage_fn<32>(stage);
    default: return stage_fn<64>(stage);
  }
}

// Kernel variant per batch size: the VALU engine holds up to 8 batch rows per
// pass (batches 9..15 take two passes); from 16 on the MFMA engine takes the
// batch in 16-row tiles.
int nb_for_batch(int B) {
  return B <= 1 ? 1 : B <= 2 ? 2 : B <= 4 ? 4 : B < kMfmaMinBatch ? 8 : B <= 16 ? 16 : B <= 32 ? 32 : 64;
}

hipError_t launch_stage(int stage, const Params& P, int l, int grid, int threads, size_t smem,
                        hipStream_t s) {
  // whole-kernel-wait launches (P.S.wait) take the full-register builds
  const void* fn = kernel_ptr(stage, nb_for_batch(P.S.B), P.S.wait != 0);
  if (!fn || stage == 0 || stage == kSMlpProj) return hipErrorInvalidValue;
  Params p = P;
  void* args[] = {&p, &l};
  return hipLaunchKernel(fn, dim3(grid), dim3(threads), args, smem, s);
}

// The persistent kernel needs every workgroup resident at once (they wait on
// each other).  The grid is the occupancy limit of an otherwise idle GPU, so
// an ordinary launch places them all; it was measured about 18 us per step
// cheaper than a cooperative launch.  If other work shares the GPU and some
// workgroups cannot start, the resident ones run into the watchdog and the
// step ends with LD_ETIMEOUT rather than hanging.
hipError_t launch_mega(const Params& P, int grid, int threads, size_t smem, hipStream_t s) {
  const void* fn = kernel_ptr(0, nb_for_batch(P.S.B));
  Params p = P;
  void* args[] = {&p};
  return hipLaunchKernel(fn, dim3(grid), dim3(threads), args, smem, s);
}

hipError_t launch_mlp_proj(int which, const Params& P, int l, int grid, int threads, size_t smem,
                           hipStream_t s) {
  const void* fn = kernel_ptr(kSMlpProj, nb_for_batch(P.S.B), P.S.wait != 0);
  if (!fn) return hipErrorInvalidValue;
  Params p = P;
  void* args[] = {&p, &l, &which};
  return hipLaunchKernel(fn, dim3(grid), dim3(threads), args, smem, s);
}

hipError_t launch_mlp_elem(int op, const Params& P, hipStream_t s) {
  const int64_t n = (int64_t)P.S.B * P.D.I;
  const int64_t blocks = (n + 255) / 256;
  const int grid = (int)(blocks < 4096 ? blocks : 4096);
  hipLaunchKernelGGL(k_mlp_elem, dim3(grid), dim3(256), 0, s, P, op, n);
  return hipGetLastError();
}

hipError_t occupancy(int stage, int nb, int threads, size_t smem, int* blocks_per_cu, bool full) {
  const void* fn = kernel_ptr(stage, nb, full);
  if (!fn) return hipErrorInvalidValue;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, fn, threads, smem);
}

hipError_t set_max_dynamic_smem(int stage, int nb, size_t smem, bool full) {
  const void* fn = kernel_ptr(stage, nb, full);
  if (!fn) return hipErrorInvalidValue;
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
}

size_t scratch_bytes() { return kScratchBytes; }

size_t attn_smem(int group, int d, int T, int max_splits) {
  return attn_smem_bytes(group, d, T, max_splits);
}

size_t best_bytes() { return kBestBytes; }

hipError_t launch_gen_normal(uint16_t* dst, int64_t n, uint64_t key, uint64_t index0, float kappa,
                             hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  const int grid = (int)(blocks < 65536 ? blocks : 65536);
  hipLaunchKernelGGL(k_gen_normal, dim3(grid), dim3(256), 0, s, dst, n, key, index0, kappa);
  return hipGetLastError();
}

hipError_t launch_poison(const PoisonRanges& r, uint16_t* kc, uint16_t* vc, const int32_t* pos,
                         int rows, int M, int L, int max_batch, int nkv, int max_seq, int d,
                         hipStream_t s) {
  hipLaunchKernelGGL(k_poison, dim3(256, r.count + 1), dim3(256), 0, s, r, kc, vc, pos, rows, M, L,
                     max_batch, nkv, max_seq, d);
  return hipGetLastError();
}

hipError_t launch_fill16(uint16_t* dst, int64_t n, uint16_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  const int grid = (int)(blocks < 65536 ? blocks : 65536);
  hipLaunchKernelGGL(k_fill16, dim3(grid), dim3(256), 0, s, dst, n, v);
  return hipGetLastError();
}

hipError_t launch_gen_kv(uint16_t* kc, uint16_t* vc, const int* len_dev, int batch, int n_kv,
                         int max_seq, int d, uint64_t kkey, uint64_t vkey, float kappa,
                         hipStream_t s) {
  const int64_t per = (int64_t)max_seq * d;
  const int64_t bx = (per + 255) / 256;
  const int gx = (int)(bx < 4096 ? bx : 4096);
  hipLaunchKernelGGL(k_gen_kv, dim3(gx, batch * n_kv), dim3(256), 0, s, kc, vc, len_dev, n_kv,
                     max_seq, d, kkey, vkey, kappa);
  return hipGetLastError();
}

}  // namespace ld
