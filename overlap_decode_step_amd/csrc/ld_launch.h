// ld_launch.h - launch wrappers exported by ld_kernels.hip to the host runtime.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ld_params.hpp"

namespace ld {

// stage: kSQkv..kSLm for the per-stage kernels, 0 for the persistent kernel.
int nb_for_batch(int B);
hipError_t launch_stage(int stage, const Params& P, int layer, int grid, int threads, size_t smem,
                        hipStream_t s);
hipError_t launch_mega(const Params& P, int grid, int threads, size_t smem, hipStream_t s);
// unfused-MLP ablation (whole-kernel-wait mode): projection GEMV `which`
// (gate, up or both) and elementwise op (silu, mul, silu-mul)
hipError_t launch_mlp_proj(int which, const Params& P, int layer, int grid, int threads,
                           size_t smem, hipStream_t s);
hipError_t launch_mlp_elem(int op, const Params& P, hipStream_t s);
// full: the whole-kernel-wait builds of the 64-row MFMA stage kernels
hipError_t occupancy(int stage, int nb, int threads, size_t smem, int* blocks_per_cu,
                     bool full = false);
hipError_t set_max_dynamic_smem(int stage, int nb, size_t smem, bool full = false);
size_t scratch_bytes();
size_t attn_smem(int group, int d, int T, int max_splits);
size_t best_bytes();

// Debug poison (see ld_set_debug): quiet NaNs into n ranges of 32-bit words
// and into the KV-cache rows the step appends (row b of the step, of
// sequence b / M, at position pos[b], in every layer and kv head).
constexpr int kPoisonRanges = 24;
struct PoisonRanges {
  uint32_t* p[kPoisonRanges];
  int64_t n[kPoisonRanges];
  int count;
};
hipError_t launch_poison(const PoisonRanges& r, uint16_t* kc, uint16_t* vc, const int32_t* pos,
                         int rows, int M, int L, int max_batch, int nkv, int max_seq, int d,
                         hipStream_t s);

hipError_t launch_gen_normal(uint16_t* dst, int64_t n, uint64_t key, uint64_t index0, float kappa,
                             hipStream_t s);
hipError_t launch_fill16(uint16_t* dst, int64_t n, uint16_t v, hipStream_t s);
// The allocation-free KV fill's device copy of the prefill lengths (a
// file-scope device array of `capacity` int32) for the current device: its
// address, looked up once per device.
hipError_t scratch_lens_ptr(int32_t** out, int* capacity);
// Write n <= capacity lengths (from host memory, passed as kernel arguments)
// and zeros after them into that array, on stream s.
hipError_t launch_put_lens(int32_t* dst, const int32_t* host_lens, int n, hipStream_t s);
hipError_t launch_gen_kv(uint16_t* kc, uint16_t* vc, const int* len_dev, int batch, int n_kv,
                         int max_seq, int d, uint64_t kkey, uint64_t vkey, float kappa,
                         hipStream_t s);

}  // namespace ld
