// HIP kernels of the paged KV-cache decode path, written for gfx950 (CDNA4, wave64).
//
// Pages cited (title, then section):
//   [Reading vLLM]  "啃透vLLM源码：从PagedAttention到连续批处理，大模型推理加速24倍的秘密"
//   [vLLM basics]   "vLLM基础：架构、推理流程与关键组件"
//   [vLLM analysis] "VLLM源码解析：高效大规模语言模型推理的技术实现"
//
// Pool layout: [num_blocks, num_heads, block_size, head_dim], so the tokens of one
// (block, head) form one contiguous chunk of block_size * head_dim elements
// (4 KiB for 16 tokens x 128 dims in fp16).
//
// Decode (partition pass).  One workgroup of kWaves wave64s per (partition, head,
// sequence).  A partition is P consecutive tokens of one sequence; its blocks are
// dealt to the waves round-robin.  Within a wave every lane loads 16 bytes per
// instruction, so one wave-wide load covers a contiguous 1 KiB of a chunk:
// kTokPerLoad token rows of kLanesPerTok lanes each.  A lane therefore always holds
// the same kVec dims of its q and of its V accumulator.  QK partial dots use
// v_dot2_f32_f16 (fp16) or fma (fp32) and are summed across the kLanesPerTok lanes
// of a row with DPP.  Each row keeps its own online-softmax state (m, l, acc) in
// registers, so the main loop needs no LDS and no barrier; rows are merged with
// shuffles and the waves through LDS once at the end.  Logits are kept in base 2:
// z = scale * log2(e) * <q, k>, weights 2^(z - m).
//
// Nothing here depends on where a block sits in the pool: the order of every
// floating-point operation is a function of logical token positions only, so
// renaming physical blocks gives bit-identical results.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_launch.h"

namespace pa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Build-time tuning knobs (defaults are the measured best on MI355X).
#ifndef PA_DECODE_WAVES
#define PA_DECODE_WAVES 8  // wave64s per decode workgroup
#endif
#ifndef PA_KV_LOADS_IN_FLIGHT
#define PA_KV_LOADS_IN_FLIGHT 8  // 16-byte K+V loads per lane issued before their use
#endif
#ifndef PA_NONTEMPORAL_KV
#define PA_NONTEMPORAL_KV 1  // 1: K/V loads carry the non-temporal (streaming) hint
#endif
#ifndef PA_WAVES_PER_EU
#define PA_WAVES_PER_EU 0  // >0: cap registers so this many waves fit per SIMD
#endif
#if PA_WAVES_PER_EU > 0
#define PA_OCCUPANCY __attribute__((amdgpu_waves_per_eu(PA_WAVES_PER_EU)))
#else
#define PA_OCCUPANCY
#endif

constexpr int kWave = 64;
constexpr int kWaves = PA_DECODE_WAVES;
constexpr int kThreads = kWave * kWaves;
constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------------
// small device helpers
// ---------------------------------------------------------------------------------

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// K/V rows are read exactly once per call.
__device__ __forceinline__ u32x4 load_kv16(const void* p) {
#if PA_NONTEMPORAL_KV
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#else
  return *reinterpret_cast<const u32x4*>(p);
#endif
}

__device__ __forceinline__ float as_float(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ f16x2 as_h2(uint32_t u) { return __builtin_bit_cast(f16x2, u); }

// DPP row operations (within rows of 16 lanes).
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

// Every row and bank enabled with bound_ctrl set, so the compiler folds the move
// into the add that consumes it (one v_add_f32 with a DPP source operand).
template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, 0xF, 0xF, true));
}

// 2^x with the hardware transcendental unit (v_exp_f32).  Softmax weights below
// 2^-126 of the running maximum may flush to zero, which changes no sum by more
// than that amount.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Sum over groups of kLanes consecutive lanes; every lane of a group receives the
// same bits (each stage adds two equal-valued operands in either order).
template <int kLanes>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(kLanes == 8 || kLanes == 16 || kLanes == 32 || kLanes == 64, "group");
  x += dpp<kDppQuadXor1>(x);
  x += dpp<kDppQuadXor2>(x);
  x += dpp<kDppRowHalfMirror>(x);
  if constexpr (kLanes >= 16) x += dpp<kDppRowMirror>(x);
  if constexpr (kLanes >= 32) x += __shfl_xor(x, 16);
  if constexpr (kLanes >= 64) x += __shfl_xor(x, 32);
  return x;
}

// Partial dot product of the lane's 16-byte slices of q and k.
template <typename T> struct Lane16;

template <> struct Lane16<_Float16> {
  static constexpr int kVec = 8;
  __device__ __forceinline__ static float dot(const u32x4& q, const u32x4& k) {
    float s = __builtin_amdgcn_fdot2(as_h2(q.x), as_h2(k.x), 0.0f, false);
    s = __builtin_amdgcn_fdot2(as_h2(q.y), as_h2(k.y), s, false);
    s = __builtin_amdgcn_fdot2(as_h2(q.z), as_h2(k.z), s, false);
    s = __builtin_amdgcn_fdot2(as_h2(q.w), as_h2(k.w), s, false);
    return s;
  }
  // acc[j] += p * v[j] in fp32
  __device__ __forceinline__ static void axpy(float p, const u32x4& v, float* acc) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f16x2 h = as_h2(w[i]);
      acc[2 * i] = __builtin_fmaf(p, static_cast<float>(h.x), acc[2 * i]);
      acc[2 * i + 1] = __builtin_fmaf(p, static_cast<float>(h.y), acc[2 * i + 1]);
    }
  }
  __device__ __forceinline__ static _Float16 from_float(float x) { return static_cast<_Float16>(x); }
};

template <> struct Lane16<float> {
  static constexpr int kVec = 4;
  __device__ __forceinline__ static float dot(const u32x4& q, const u32x4& k) {
    float s = as_float(q.x) * as_float(k.x);
    s = __builtin_fmaf(as_float(q.y), as_float(k.y), s);
    s = __builtin_fmaf(as_float(q.z), as_float(k.z), s);
    s = __builtin_fmaf(as_float(q.w), as_float(k.w), s);
    return s;
  }
  __device__ __forceinline__ static void axpy(float p, const u32x4& v, float* acc) {
    acc[0] = __builtin_fmaf(p, as_float(v.x), acc[0]);
    acc[1] = __builtin_fmaf(p, as_float(v.y), acc[1]);
    acc[2] = __builtin_fmaf(p, as_float(v.z), acc[2]);
    acc[3] = __builtin_fmaf(p, as_float(v.w), acc[3]);
  }
  __device__ __forceinline__ static float from_float(float x) { return x; }
};

// Compile-time geometry of one (dtype, head_dim, block_size) instance.
template <typename T, int D, int BS>
struct Geometry {
  static constexpr int kVec = Lane16<T>::kVec;             // elements per 16-byte load
  static constexpr int kLanesPerTok = D / kVec;            // lanes covering one token row
  static constexpr int kTokPerLoad = kWave / kLanesPerTok; // token rows per wave-wide load
  static constexpr int kLoads = BS / kTokPerLoad;          // loads per (block, head) chunk
  // blocks fetched together per wave: PA_KV_LOADS_IN_FLIGHT 16-byte loads per lane
  static constexpr int kUnroll =
      2 * kLoads >= PA_KV_LOADS_IN_FLIGHT ? 1 : PA_KV_LOADS_IN_FLIGHT / (2 * kLoads);
  static_assert(D % kVec == 0 && kWave % kLanesPerTok == 0, "head_dim");
  static_assert(BS % kTokPerLoad == 0, "block_size");
};

// Online-softmax state of one token row of one wave.
template <int kVec>
struct RowState {
  float m;          // running max of base-2 logits (-inf before the first token)
  float l;          // sum of 2^(z - m)
  float acc[kVec];  // sum of 2^(z - m) * v over this lane's kVec dims
};

// Fold one block of one head into the row state.  kTail: only the first n_valid
// tokens of the block are live; the others are skipped (never multiplied by zero,
// because the slots past the end may hold anything, NaN included).
template <typename T, int D, int BS, bool kTail>
__device__ __forceinline__ void fold_block(RowState<Geometry<T, D, BS>::kVec>& st,
                                           const u32x4& q, const u32x4* kr,
                                           const u32x4* vr, float scale_log2,
                                           int row, int n_valid) {
  using G = Geometry<T, D, BS>;
  float z[G::kLoads];
#pragma unroll
  for (int i = 0; i < G::kLoads; ++i) {
    z[i] = group_sum<G::kLanesPerTok>(Lane16<T>::dot(q, kr[i])) * scale_log2;
    if constexpr (kTail) {
      if (i * G::kTokPerLoad + row >= n_valid) z[i] = -INFINITY;
    }
  }
  float top = z[0];
#pragma unroll
  for (int i = 1; i < G::kLoads; ++i) top = fmaxf(top, z[i]);
  const float m_new = fmaxf(st.m, top);
  float alpha;
  if constexpr (kTail) {
    alpha = (m_new == -INFINITY) ? 1.0f : fast_exp2(st.m - m_new);
  } else {
    alpha = fast_exp2(st.m - m_new);  // m_new is finite: every token of the block is live
  }
  st.l *= alpha;
#pragma unroll
  for (int j = 0; j < G::kVec; ++j) st.acc[j] *= alpha;
#pragma unroll
  for (int i = 0; i < G::kLoads; ++i) {
    if constexpr (kTail) {
      if (i * G::kTokPerLoad + row >= n_valid) continue;
    }
    const float p = fast_exp2(z[i] - m_new);
    st.l += p;
    Lane16<T>::axpy(p, vr[i], st.acc);
  }
  st.m = m_new;
}

// Merge state b into a by the log-sum-exp rule; symmetric in (a, b) bit for bit.
template <int kVec>
__device__ __forceinline__ void merge_state(RowState<kVec>& a, float m_b, float l_b,
                                            const float* acc_b) {
  const float m = fmaxf(a.m, m_b);
  const float fa = (a.m == -INFINITY) ? 0.0f : fast_exp2(a.m - m);
  const float fb = (m_b == -INFINITY) ? 0.0f : fast_exp2(m_b - m);
  a.l = a.l * fa + l_b * fb;
#pragma unroll
  for (int j = 0; j < kVec; ++j) a.acc[j] = a.acc[j] * fa + acc_b[j] * fb;
  a.m = m;
}

// Fold this wave's blocks of one (partition, head) into its row state.  Lane j of
// `ids` holds the physical id of the wave's j-th block (the first kWave of them);
// a longer list is fetched kWave at a time from `my_table` (stride kWaves).
template <typename T, int D, int BS>
__device__ __forceinline__ void attend_blocks(RowState<Geometry<T, D, BS>::kVec>& st,
                                              const u32x4& q, int ids, const int* my_table,
                                              const T* k_head, const T* v_head,
                                              size_t block_stride, int lane_off, int lane,
                                              int row, int n_mine, int n_full, int tail_valid,
                                              float scale_log2) {
  using G = Geometry<T, D, BS>;
  for (int base = 0; base < n_mine; base += kWave) {
    if (base > 0) {
      const int idx = base + lane;
      ids = idx < n_mine ? my_table[idx * kWaves] : 0;
    }
    const int chunk_full = min(max(n_full - base, 0), kWave);
    int j = 0;
    // kUnroll full blocks per iteration, all loads issued before use
    for (; j + G::kUnroll <= chunk_full; j += G::kUnroll) {
      u32x4 kr[G::kUnroll][G::kLoads];
      u32x4 vr[G::kUnroll][G::kLoads];
#pragma unroll
      for (int u = 0; u < G::kUnroll; ++u) {
        const int phys = __builtin_amdgcn_readlane(ids, j + u);
        const T* kp = k_head + static_cast<size_t>(phys) * block_stride + lane_off;
#pragma unroll
        for (int i = 0; i < G::kLoads; ++i) kr[u][i] = load_kv16(kp + i * G::kTokPerLoad * D);
      }
#pragma unroll
      for (int u = 0; u < G::kUnroll; ++u) {
        const int phys = __builtin_amdgcn_readlane(ids, j + u);
        const T* vp = v_head + static_cast<size_t>(phys) * block_stride + lane_off;
#pragma unroll
        for (int i = 0; i < G::kLoads; ++i) vr[u][i] = load_kv16(vp + i * G::kTokPerLoad * D);
      }
#pragma unroll
      for (int u = 0; u < G::kUnroll; ++u)
        fold_block<T, D, BS, false>(st, q, kr[u], vr[u], scale_log2, row, BS);
    }
    // remaining full blocks of this chunk, one at a time
    for (; j < chunk_full; ++j) {
      u32x4 kr[G::kLoads];
      u32x4 vr[G::kLoads];
      const int phys = __builtin_amdgcn_readlane(ids, j);
      const T* kp = k_head + static_cast<size_t>(phys) * block_stride + lane_off;
      const T* vp = v_head + static_cast<size_t>(phys) * block_stride + lane_off;
#pragma unroll
      for (int i = 0; i < G::kLoads; ++i) kr[i] = load_kv16(kp + i * G::kTokPerLoad * D);
#pragma unroll
      for (int i = 0; i < G::kLoads; ++i) vr[i] = load_kv16(vp + i * G::kTokPerLoad * D);
      fold_block<T, D, BS, false>(st, q, kr, vr, scale_log2, row, BS);
    }
    // the partly filled last block of the partition, if this chunk holds it
    if (n_mine > n_full && base + j == n_full && j < kWave && base + j < n_mine) {
      u32x4 kr[G::kLoads];
      u32x4 vr[G::kLoads];
      const int phys = __builtin_amdgcn_readlane(ids, j);
      const T* kp = k_head + static_cast<size_t>(phys) * block_stride + lane_off;
      const T* vp = v_head + static_cast<size_t>(phys) * block_stride + lane_off;
#pragma unroll
      for (int i = 0; i < G::kLoads; ++i) kr[i] = load_kv16(kp + i * G::kTokPerLoad * D);
#pragma unroll
      for (int i = 0; i < G::kLoads; ++i) vr[i] = load_kv16(vp + i * G::kTokPerLoad * D);
      fold_block<T, D, BS, true>(st, q, kr, vr, scale_log2, row, tail_valid);
    }
  }
}

// ---------------------------------------------------------------------------------
// decode, partition pass
// grid (max partitions, heads, seqs), kThreads threads
// ---------------------------------------------------------------------------------

template <typename T, int D, int BS>
__global__ __launch_bounds__(kThreads) PA_OCCUPANCY void decode_partitions_kernel(DecodeParams prm) {
  using G = Geometry<T, D, BS>;
  constexpr int kVec = G::kVec;

  const int part = blockIdx.x;
  const int head = blockIdx.y;
  const int seq = blockIdx.z;
  const int P = prm.partition_tokens;
  const int tok_begin = part * P;
  const int blk_begin = tok_begin / BS;  // P is a multiple of BS

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int row = lane / G::kLanesPerTok;
  const int col = lane % G::kLanesPerTok;

  // Issued together, before anything waits on memory: the context length, the
  // query row and the ids of this wave's first kWave blocks.  The ids are bounded
  // by the table row, not by the context (entries past the context are read but
  // never used), so the K/V stream waits on one dependent load instead of two.
  const int* table = prm.block_tables + static_cast<size_t>(seq) * prm.max_blocks_per_seq;
  const int* my_table = table + blk_begin + wave;
  const int ids0 = blk_begin + wave + lane * kWaves < prm.max_blocks_per_seq ? my_table[lane * kWaves] : 0;
  const u32x4 q = load16(static_cast<const T*>(prm.query) +
                         (static_cast<size_t>(seq) * prm.num_heads + head) * D + col * kVec);
  const int ctx = prm.context_lens[seq];
  T* out_row = static_cast<T*>(prm.out) + (static_cast<size_t>(seq) * prm.num_heads + head) * D;

  if (tok_begin >= ctx) {
    if (part == 0) {  // empty sequence: the output is zero
      for (int d = threadIdx.x; d < D; d += kThreads) out_row[d] = Lane16<T>::from_float(0.0f);
    }
    return;
  }
  const int tok_end = min(ctx, tok_begin + P);
  const int full_end = tok_end / BS;  // blocks whose every token is live
  const int blk_end = (tok_end + BS - 1) / BS;

  const size_t block_stride = static_cast<size_t>(prm.num_heads) * BS * D;  // elements
  const T* k_head = static_cast<const T*>(prm.key_cache) + static_cast<size_t>(head) * BS * D;
  const T* v_head = static_cast<const T*>(prm.value_cache) + static_cast<size_t>(head) * BS * D;
  const int lane_off = row * D + col * kVec;  // element offset of this lane in load 0
  const float scale_log2 = prm.scale * kLog2e;

  // This wave owns logical blocks blk_begin + wave + j * kWaves, j < n_mine; the
  // last of them may be partly filled.
  const int n_total = blk_end - blk_begin;
  const int n_mine = n_total > wave ? (n_total - wave + kWaves - 1) / kWaves : 0;
  const int n_full = full_end - blk_begin > wave ? (full_end - blk_begin - wave + kWaves - 1) / kWaves : 0;
  const int tail_valid = tok_end - (blk_begin + wave + n_full * kWaves) * BS;

  RowState<kVec> st;
  st.m = -INFINITY;
  st.l = 0.0f;
#pragma unroll
  for (int j = 0; j < kVec; ++j) st.acc[j] = 0.0f;
  attend_blocks<T, D, BS>(st, q, ids0, my_table, k_head, v_head, block_stride, lane_off, lane, row,
                          n_mine, n_full, tail_valid, scale_log2);

  // merge the token rows of the wave (lanes with the same col)
#pragma unroll
  for (int off = G::kLanesPerTok; off < kWave; off <<= 1) {
    const float m_o = __shfl_xor(st.m, off);
    const float l_o = __shfl_xor(st.l, off);
    float acc_o[kVec];
#pragma unroll
    for (int j = 0; j < kVec; ++j) acc_o[j] = __shfl_xor(st.acc[j], off);
    merge_state<kVec>(st, m_o, l_o, acc_o);
  }

  // merge the waves through LDS, in wave order
  __shared__ float s_m[kWaves];
  __shared__ float s_l[kWaves];
  __shared__ float s_o[kWaves][D];
  if (row == 0) {
#pragma unroll
    for (int j = 0; j < kVec; ++j) s_o[wave][col * kVec + j] = st.acc[j];
    if (col == 0) {
      s_m[wave] = st.m;
      s_l[wave] = st.l;
    }
  }
  __syncthreads();

  const bool single = ctx <= P;
  for (int d = threadIdx.x; d < D; d += kThreads) {
    float m = s_m[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) m = fmaxf(m, s_m[w]);
    float l = 0.0f;
    float o = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = (s_m[w] == -INFINITY) ? 0.0f : fast_exp2(s_m[w] - m);
      l = l + s_l[w] * f;
      o = o + s_o[w][d] * f;
    }
    if (single) {
      out_row[d] = Lane16<T>::from_float(o / l);
    } else {
      const size_t slot = (static_cast<size_t>(seq) * prm.num_heads + head) * prm.num_partitions + part;
      prm.ws_o[slot * D + d] = o;
      if (d == 0) {
        prm.ws_m[slot] = m;
        prm.ws_l[slot] = l;
      }
    }
  }
}

// ---------------------------------------------------------------------------------
// decode, reduce pass: grid (heads, seqs), D threads
// ---------------------------------------------------------------------------------

template <typename T, int D>
__global__ __launch_bounds__(D) void decode_reduce_kernel(ReduceParams prm) {
  const int head = blockIdx.x;
  const int seq = blockIdx.y;
  const int ctx = prm.context_lens[seq];
  const int P = prm.partition_tokens;
  const int np = (ctx + P - 1) / P;
  if (np <= 1) return;  // written directly by the partition pass
  const int d = threadIdx.x;
  const size_t base = (static_cast<size_t>(seq) * prm.num_heads + head) * prm.num_partitions;

  float m = -INFINITY;
  for (int p = 0; p < np; ++p) m = fmaxf(m, prm.ws_m[base + p]);
  float l = 0.0f;
  float o = 0.0f;
  for (int p = 0; p < np; ++p) {
    const float f = fast_exp2(prm.ws_m[base + p] - m);
    l = l + prm.ws_l[base + p] * f;
    o = o + prm.ws_o[(base + p) * D + d] * f;
  }
  T* out_row = static_cast<T*>(prm.out) + (static_cast<size_t>(seq) * prm.num_heads + head) * D;
  out_row[d] = Lane16<T>::from_float(o / l);
}

// ---------------------------------------------------------------------------------
// cache append: one thread per 16 bytes of a (token, head) row, K and V
// ---------------------------------------------------------------------------------

__global__ __launch_bounds__(256) void cache_append_kernel(AppendParams prm) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int chunks = prm.row_bytes / 16;
  const int64_t total = static_cast<int64_t>(prm.num_tokens) * prm.num_heads * chunks;
  if (idx >= total) return;
  const int c = static_cast<int>(idx % chunks);
  const int64_t th = idx / chunks;  // token * heads + head
  const int h = static_cast<int>(th % prm.num_heads);
  const int i = static_cast<int>(th / prm.num_heads);
  const int slot = prm.slot_mapping[i];
  if (slot < 0) return;
  const int b = slot / prm.block_size;
  const int o = slot % prm.block_size;
  const size_t dst = ((static_cast<size_t>(b) * prm.num_heads + h) * prm.block_size + o) *
                         static_cast<size_t>(prm.row_bytes) + static_cast<size_t>(c) * 16;
  const size_t src = static_cast<size_t>(th) * prm.row_bytes + static_cast<size_t>(c) * 16;
  const u32x4 kv = load16(static_cast<const char*>(prm.key) + src);
  const u32x4 vv = load16(static_cast<const char*>(prm.value) + src);
  *reinterpret_cast<u32x4*>(static_cast<char*>(prm.key_cache) + dst) = kv;
  *reinterpret_cast<u32x4*>(static_cast<char*>(prm.value_cache) + dst) = vv;
}

// ---------------------------------------------------------------------------------
// block copy: grid (pairs, chunk groups of a block); 16 bytes per thread per step
// ---------------------------------------------------------------------------------

__global__ __launch_bounds__(256) void block_copy_kernel(CopyParams prm) {
  const int pair = blockIdx.x;
  const int src = prm.block_pairs[2 * pair];
  const int dst = prm.block_pairs[2 * pair + 1];
  const int64_t chunks = prm.block_bytes / 16;
  const char* ks = static_cast<const char*>(prm.key_cache) + static_cast<size_t>(src) * prm.block_bytes;
  const char* vs = static_cast<const char*>(prm.value_cache) + static_cast<size_t>(src) * prm.block_bytes;
  char* kd = static_cast<char*>(prm.key_cache) + static_cast<size_t>(dst) * prm.block_bytes;
  char* vd = static_cast<char*>(prm.value_cache) + static_cast<size_t>(dst) * prm.block_bytes;
  for (int64_t c = static_cast<int64_t>(blockIdx.y) * blockDim.x + threadIdx.x; c < chunks;
       c += static_cast<int64_t>(gridDim.y) * blockDim.x) {
    const u32x4 k = load16(ks + c * 16);
    const u32x4 v = load16(vs + c * 16);
    *reinterpret_cast<u32x4*>(kd + c * 16) = k;
    *reinterpret_cast<u32x4*>(vd + c * 16) = v;
  }
}

// ---------------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------------

template <typename T, int D, int BS>
static hipError_t launch_partitions_t(const DecodeParams& prm, hipStream_t stream) {
  dim3 grid(prm.num_partitions, prm.num_heads, prm.num_seqs);
  hipLaunchKernelGGL((decode_partitions_kernel<T, D, BS>), grid, dim3(kThreads), 0, stream, prm);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_partitions_d(const DecodeParams& prm, int block_size, hipStream_t stream) {
  switch (block_size) {
    case 8: return launch_partitions_t<T, D, 8>(prm, stream);
    case 16: return launch_partitions_t<T, D, 16>(prm, stream);
    case 32: return launch_partitions_t<T, D, 32>(prm, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
static hipError_t launch_partitions_dt(const DecodeParams& prm, int head_dim, int block_size,
                                       hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_partitions_d<T, 64>(prm, block_size, stream);
    case 128: return launch_partitions_d<T, 128>(prm, block_size, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_partitions(const DecodeParams& prm, bool f16, int head_dim,
                                    int block_size, hipStream_t stream) {
  return f16 ? launch_partitions_dt<_Float16>(prm, head_dim, block_size, stream)
             : launch_partitions_dt<float>(prm, head_dim, block_size, stream);
}

template <typename T>
static hipError_t launch_reduce_t(const ReduceParams& prm, int head_dim, hipStream_t stream) {
  dim3 grid(prm.num_heads, prm.num_seqs);
  switch (head_dim) {
    case 64:
      hipLaunchKernelGGL((decode_reduce_kernel<T, 64>), grid, dim3(64), 0, stream, prm);
      break;
    case 128:
      hipLaunchKernelGGL((decode_reduce_kernel<T, 128>), grid, dim3(128), 0, stream, prm);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_reduce(const ReduceParams& prm, bool f16, int head_dim, hipStream_t stream) {
  return f16 ? launch_reduce_t<_Float16>(prm, head_dim, stream)
             : launch_reduce_t<float>(prm, head_dim, stream);
}

hipError_t launch_cache_append(const AppendParams& prm, hipStream_t stream) {
  const int64_t total = static_cast<int64_t>(prm.num_tokens) * prm.num_heads * (prm.row_bytes / 16);
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(cache_append_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, prm);
  return hipGetLastError();
}

hipError_t launch_block_copy(const CopyParams& prm, hipStream_t stream) {
  const int64_t chunks = prm.block_bytes / 16;
  int64_t gy = (chunks + 256 * 4 - 1) / (256 * 4);  // about 4 chunks per thread
  if (gy < 1) gy = 1;
  if (gy > 1024) gy = 1024;
  hipLaunchKernelGGL(block_copy_kernel, dim3(prm.num_pairs, static_cast<unsigned>(gy)), dim3(256), 0,
                     stream, prm);
  return hipGetLastError();
}

}  // namespace pa
