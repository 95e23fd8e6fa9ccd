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
// Decode (partition pass).  One workgroup of W wave64s (8 or 16, chosen per launch)
// per (partition, head, sequence).  A partition is P consecutive tokens of one sequence; its blocks are
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
#ifndef PA_KV_LOADS_IN_FLIGHT
#define PA_KV_LOADS_IN_FLIGHT 8  // 16-byte K+V loads per lane issued before their use
#endif
#ifndef PA_KV_LOADS_IN_FLIGHT_WIDE
#define PA_KV_LOADS_IN_FLIGHT_WIDE 16  // the same for the 16-wave decode workgroups
#endif
#ifndef PA_NONTEMPORAL_KV
#define PA_NONTEMPORAL_KV 1  // 1: K/V loads carry the non-temporal (streaming) hint
#endif
#ifndef PA_KV_BUFFER_AUX
#define PA_KV_BUFFER_AUX -1  // >= 0: K/V read by buffer loads with this cache-policy word
#endif
#ifndef PA_HEADS_PER_UNIT
#define PA_HEADS_PER_UNIT 1  // 2: heads a wave folds per unit when a (block, head) chunk is 4 KiB
#endif
#ifndef PA_MAX_LOADS_PER_UNIT
#define PA_MAX_LOADS_PER_UNIT 8  // K (and V) loads per lane for one unit of a block
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
constexpr int kWavesNarrow = kDecodeWavesNarrow;  // the two decode workgroup sizes (pa_launch.h)
constexpr int kWavesWide = kDecodeWavesWide;
constexpr float kLog2e = 1.4426950408889634f;

// Tokens (and queries) per matrix-core tile of the shared-prefix decode.  The prefix
// pass reads a sequence's shared prefix in whole tiles: with blocks of 8 tokens a prefix
// that ends inside a tile is rounded down to whole tiles, and the pass after the prefix
// starts at that rounded length (with blocks of 16 tokens or more every prefix is a whole
// number of tiles already).  Every reader of the prefix lengths applies tiled_prefix.
constexpr int kTile = 16;
__device__ __forceinline__ int tiled_prefix(int prefix_len) { return prefix_len & ~(kTile - 1); }

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

// Load i of a lane in one unit of a (block, head) chunk: `unit` is the unit's first
// element (the same in every lane), `elem` this load's element offset in it.
template <typename T, int kUnitBytes>
__device__ __forceinline__ u32x4 load_unit16(const T* unit, int elem) {
#if PA_KV_BUFFER_AUX >= 0
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(unit), 0, kUnitBytes, 0x00020000);
  return __builtin_amdgcn_raw_buffer_load_b128(r, elem * static_cast<int>(sizeof(T)), 0, PA_KV_BUFFER_AUX);
#else
  return load_kv16(unit + elem);
#endif
}

__device__ __forceinline__ void store16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }

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

constexpr int pow2_ceil(int x) {
  int p = 1;
  while (p < x) p *= 2;
  return p;
}

// Compile-time geometry of one (dtype, head_dim, block_size) instance.  A token row
// is spread over kLanesPerTok lanes (a power of two), of which the first kActive hold
// 16 bytes of it; when D / kVec is not a power of two the other lanes of the row
// are idle (their scores are masked to zero and their sums never leave the lane).
// A unit is the run of consecutive tokens of one block that a wave folds at once:
// the whole block, or a slice of it when the block would need more than
// PA_MAX_LOADS_PER_UNIT loads.
template <typename T, int D, int BS>
struct Geometry {
  static constexpr int kVec = Lane16<T>::kVec;             // elements per 16-byte load
  static constexpr int kActive = D / kVec;                 // lanes with data in a row
  static constexpr int kLanesPerTok = pow2_ceil(kActive);  // lanes per token row
  static constexpr int kTokPerLoad = kWave / kLanesPerTok; // token rows per wave-wide load
  static constexpr int kUnitTok =
      BS < kTokPerLoad * PA_MAX_LOADS_PER_UNIT ? BS : kTokPerLoad * PA_MAX_LOADS_PER_UNIT;
  static constexpr int kUnitsPerBlock = BS / kUnitTok;
  static constexpr int kLoads = kUnitTok / kTokPerLoad;    // loads per unit (K, and V)
  // whole units a wave fetches together, all their loads issued before the first fold,
  // for `in_flight` 16-byte K+V loads per lane (at least one unit)
  static constexpr int units_in_flight(int in_flight) {
    return 2 * kLoads >= in_flight ? 1 : in_flight / (2 * kLoads);
  }
  // Heads of one block a wave may fold as one unit (PA_HEADS_PER_UNIT): the chunks of
  // adjacent heads are adjacent in the pool, so two 4 KiB chunks are one contiguous
  // 8 KiB run per unit of K (and of V), the run a 32-token block of one head gives.
  // Measured on MI355X (fp16, 32 heads x 128, the same 96 contexts U[300, 2048]): one
  // head per unit at block size 16 streams 6.59 TB/s, at block size 32 6.72 TB/s; but
  // two heads per unit at block size 16 took 351-353 us against 292 us (128 VGPRs and
  // spilled pointers at 16 waves; half the workgroups), so the default is one.
  static constexpr int kMaxHeadsPerUnit =
      (kUnitsPerBlock == 1 && BS * D * static_cast<int>(sizeof(T)) == 4096) ? PA_HEADS_PER_UNIT : 1;
  static_assert(D % kVec == 0 && kLanesPerTok <= kWave, "head_dim");
  static_assert(BS % kUnitTok == 0 && kUnitTok % kTokPerLoad == 0, "block_size");
};

// Online-softmax state of one token row of one wave.
template <int kVec>
struct RowState {
  float m;          // running max of base-2 logits (-inf before the first token)
  float l;          // sum of 2^(z - m)
  float acc[kVec];  // sum of 2^(z - m) * v over this lane's kVec dims
};

// Fold one unit of one head into the row state.  kTail: only the first n_valid
// tokens of the unit are live; the others are skipped (never multiplied by zero,
// because the slots past the end may hold anything, NaN included).  `active`: this
// lane holds data of its row (false only on the idle lanes of a padded row).
template <typename T, int D, int BS, bool kTail>
__device__ __forceinline__ void fold_unit(RowState<Geometry<T, D, BS>::kVec>& st,
                                          const u32x4& q, const u32x4* kr,
                                          const u32x4* vr, float scale_log2,
                                          int row, bool active, int n_valid) {
  using G = Geometry<T, D, BS>;
  float z[G::kLoads];
#pragma unroll
  for (int i = 0; i < G::kLoads; ++i) {
    float part = Lane16<T>::dot(q, kr[i]);
    if constexpr (G::kActive != G::kLanesPerTok) part = active ? part : 0.0f;
    z[i] = group_sum<G::kLanesPerTok>(part) * scale_log2;
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
    alpha = fast_exp2(st.m - m_new);  // m_new is finite: every token of the unit is live
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

// Element offset of unit u in the K (or V) pool, relative to the head's chunk of
// block 0, for physical block `phys`.
template <typename T, int D, int BS>
__device__ __forceinline__ size_t unit_offset(int phys, int u, size_t block_stride) {
  using G = Geometry<T, D, BS>;
  size_t off = static_cast<size_t>(phys) * block_stride;
  if constexpr (G::kUnitsPerBlock > 1) off += static_cast<size_t>(u % G::kUnitsPerBlock) * G::kUnitTok * D;
  return off;
}

// The newest token's row when the append is fused into the decode (pa_decode_append).
// `on` only in the workgroup whose partition ends with that token; the wave that owns
// the partition's last unit reads the row (k, v: this lane's 16 bytes of it) in place of
// the pool slot among that unit's loads.  The row reaches the pools through a
// workgroup of its own (store_new_row), so no decode workgroup waits on a store.
template <typename T>
struct NewRow {
  bool on;
  const T* k;  // this lane's 16 bytes of the first head's row; head j at + j * D
  const T* v;
};

// Fold this wave's units of one (partition, HU heads) into its row states.  The wave
// owns units first_unit + j * W (W waves per workgroup), j < n_mine; the first n_full
// are whole.  Lane j of `ids` holds the physical block of the wave's j-th unit (the
// first kWave of them); a longer list is fetched kWave at a time from the table.
// With HU > 1 a unit spans the same tokens of HU adjacent heads, one contiguous run of
// the pool: loads [j * kLoads, (j + 1) * kLoads) are head j's, folded into st[j] in the
// same order as with one head per unit, so the result does not depend on HU.
// With nr.on, the partition's last unit is always folded as the partly filled one
// and its last live token comes from nr (the same bits the append would have stored,
// so the result is the same as appending first and decoding after).
template <typename T, int D, int BS, int W, int HU>
__device__ __forceinline__ void attend_units(RowState<Geometry<T, D, BS>::kVec> (&st)[HU],
                                             const u32x4 (&q)[HU], int ids, const int* table,
                                             int first_unit, const T* k_head, const T* v_head,
                                             size_t block_stride, int lane_off, int lane,
                                             int row, bool active, int n_mine, int n_full,
                                             int tail_valid, float scale_log2, NewRow<T>& nr) {
  using G = Geometry<T, D, BS>;
  static_assert(HU == 1 || G::kUnitsPerBlock == 1, "heads share a unit only when the unit is the block");
  constexpr int kL = HU * G::kLoads;  // loads per unit of K (and of V)
  constexpr int kUnitBytes = HU * G::kUnitTok * D * static_cast<int>(sizeof(T));
  // Loads in flight per lane: 8 in the 8-wave workgroups, 16 in the 16-wave ones (two
  // 8-load units at block size 16, fp16 D 128).  The 16-wave instance holds one workgroup
  // per CU at either depth (74 or 89 VGPRs), and the deeper one streams 0.6-1.1 % faster
  // on batches of 96 and 256 sequences U[300, 2048] (fp16; block size 8 and 16, D 96 and
  // 128) and 1.8 % at D 64 with blocks of 32, the same on short contexts (MI355X, same
  // box, interleaved builds); in the 8-wave instance the extra registers would cost a
  // third of its workgroups per CU.  The fold order is the same, so are the results.
  constexpr int kInFlight = W == kWavesWide ? PA_KV_LOADS_IN_FLIGHT_WIDE : PA_KV_LOADS_IN_FLIGHT;
  constexpr int kUnroll = HU == 1 ? G::units_in_flight(kInFlight) : 1;
  // element offset of this lane's load i in a unit: head i / kLoads, rows (i % kLoads)
  auto elem = [&](int i) {
    return (i / G::kLoads) * (BS * D) + (i % G::kLoads) * G::kTokPerLoad * D + lane_off;
  };
  auto fold_whole = [&](const u32x4* kr, const u32x4* vr) {
#pragma unroll
    for (int h = 0; h < HU; ++h)
      fold_unit<T, D, BS, false>(st[h], q[h], kr + h * G::kLoads, vr + h * G::kLoads, scale_log2, row, active,
                                 G::kUnitTok);
  };
  for (int base = 0; base < n_mine; base += kWave) {
    if (base > 0) {
      const int idx = base + lane;
      ids = idx < n_mine ? table[(first_unit + idx * W) / G::kUnitsPerBlock] : 0;
    }
    const int chunk_full = min(max(n_full - base, 0), kWave);
    int j = 0;
    // kUnroll whole units per iteration, all loads issued before use
    for (; j + kUnroll <= chunk_full; j += kUnroll) {
      u32x4 kr[kUnroll][kL];
      u32x4 vr[kUnroll][kL];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int phys = __builtin_amdgcn_readlane(ids, j + u);
        const size_t off = unit_offset<T, D, BS>(phys, first_unit + (base + j + u) * W, block_stride);
#pragma unroll
        for (int i = 0; i < kL; ++i) kr[u][i] = load_unit16<T, kUnitBytes>(k_head + off, elem(i));
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int phys = __builtin_amdgcn_readlane(ids, j + u);
        const size_t off = unit_offset<T, D, BS>(phys, first_unit + (base + j + u) * W, block_stride);
#pragma unroll
        for (int i = 0; i < kL; ++i) vr[u][i] = load_unit16<T, kUnitBytes>(v_head + off, elem(i));
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) fold_whole(kr[u], vr[u]);
    }
    // remaining whole units of this chunk, one at a time
    for (; j < chunk_full; ++j) {
      u32x4 kr[kL];
      u32x4 vr[kL];
      const int phys = __builtin_amdgcn_readlane(ids, j);
      const size_t off = unit_offset<T, D, BS>(phys, first_unit + (base + j) * W, block_stride);
#pragma unroll
      for (int i = 0; i < kL; ++i) kr[i] = load_unit16<T, kUnitBytes>(k_head + off, elem(i));
#pragma unroll
      for (int i = 0; i < kL; ++i) vr[i] = load_unit16<T, kUnitBytes>(v_head + off, elem(i));
      fold_whole(kr, vr);
    }
    // the partly filled last unit of the partition, if this chunk holds it
    if (n_mine > n_full && base + j == n_full && j < kWave && base + j < n_mine) {
      u32x4 kr[kL];
      u32x4 vr[kL];
      const int phys = __builtin_amdgcn_readlane(ids, j);
      const size_t off = unit_offset<T, D, BS>(phys, first_unit + (base + j) * W, block_stride);
      // with nr.on, token tail_valid - 1 of this unit is the new one: the lanes of its
      // row load it from the new rows (every head of the unit) instead of the pool
      // slot, which the store workgroups write meanwhile.  The lanes of rows past the
      // last live token load nothing (the fold below never uses those registers), so
      // the slots past the context cost no HBM traffic.
      const int r_new = tail_valid - 1;
      const int i_new = nr.on ? r_new / G::kTokPerLoad : -1;
      const bool mine = row == r_new % G::kTokPerLoad;
      const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < kL; ++i) {
        const bool fresh = i % G::kLoads == i_new && mine;
        const bool live = (i % G::kLoads) * G::kTokPerLoad + row < tail_valid;
        kr[i] = live ? load_kv16(fresh ? nr.k + (i / G::kLoads) * D : k_head + off + elem(i)) : zero;
      }
#pragma unroll
      for (int i = 0; i < kL; ++i) {
        const bool fresh = i % G::kLoads == i_new && mine;
        const bool live = (i % G::kLoads) * G::kTokPerLoad + row < tail_valid;
        vr[i] = live ? load_kv16(fresh ? nr.v + (i / G::kLoads) * D : v_head + off + elem(i)) : zero;
      }
      if (tail_valid == G::kUnitTok) {  // only with nr.on: the new token closes its unit,
        fold_whole(kr, vr);             // folded whole as without it
      } else {
#pragma unroll
        for (int h = 0; h < HU; ++h)
          fold_unit<T, D, BS, true>(st[h], q[h], kr + h * G::kLoads, vr + h * G::kLoads, scale_log2, row, active,
                                    tail_valid);
      }
    }
  }
}

// Fold the prefix states of (seq, head) -- partitions of the first `start` tokens,
// left in the workspace by the prefix pass -- into the state (m, l, o) of dim d.
__device__ __forceinline__ void fold_prefix_states(const DecodeParams& prm, int seq, int head,
                                                   int start, int d, int D, float& m, float& l,
                                                   float& o) {
  const int Pp = prm.prefix_partition_tokens;
  const int np_prefix = (start + Pp - 1) / Pp;
  const size_t base = (static_cast<size_t>(seq) * prm.num_heads + head) * prm.slots_per_pair;
  for (int p = 0; p < np_prefix; ++p) {
    const float mp = prm.ws_m[base + p];
    const float mm = fmaxf(m, mp);
    const float fa = (m == -INFINITY) ? 0.0f : fast_exp2(m - mm);
    const float fb = fast_exp2(mp - mm);
    l = l * fa + prm.ws_l[base + p] * fb;
    o = o * fa + prm.ws_o[(base + p) * D + d] * fb;
    m = mm;
  }
}

// pa_decode_append: the store workgroup of sequence `seq` (one of the grid's extra
// z-slices, dispatched after every decode workgroup, so they run in the launch's
// tail) writes the sequence's new K and V row, every head, into the slot of its position
// context_lens[seq] - 1.  The decode workgroups fold that row from new_key /
// new_value, not from the pools: they never read that slot, so the two never wait
// on each other.
// The pools are written only by pa_decode_append, whose caller passes them writable.
template <typename T, int D, int BS, int kThreads>
__device__ __forceinline__ void store_new_row(const DecodeParams& prm, int seq) {
  const int ctx = prm.context_lens[seq];
  if (ctx <= 0) return;
  const int pos = ctx - 1;
  const int blk = prm.block_tables[static_cast<size_t>(seq) * prm.max_blocks_per_seq + pos / BS];
  constexpr int kChunks = D * static_cast<int>(sizeof(T)) / 16;  // 16-byte chunks per row
  constexpr int kElems = 16 / static_cast<int>(sizeof(T));
  const size_t src_row = static_cast<size_t>(seq) * prm.num_heads;
  const size_t dst_row = static_cast<size_t>(blk) * prm.num_heads;
  T* k_pool = static_cast<T*>(const_cast<void*>(prm.key_cache));
  T* v_pool = static_cast<T*>(const_cast<void*>(prm.value_cache));
  for (int t = threadIdx.x; t < prm.num_heads * kChunks; t += kThreads) {
    const int h = t / kChunks;
    const int c = t - h * kChunks;
    const size_t src = (src_row + h) * D + static_cast<size_t>(c) * kElems;
    const size_t dst = ((dst_row + h) * BS + pos % BS) * D + static_cast<size_t>(c) * kElems;
    store16(k_pool + dst, load16(static_cast<const T*>(prm.new_key) + src));
    store16(v_pool + dst, load16(static_cast<const T*>(prm.new_value) + src));
  }
}

// Extra rows appended by trailing workgroups of a decode launch: rows [first, first +
// count) of extra_key / extra_value go to their slots, every head, K and V.  Each
// thread moves 16-byte chunks, kBatch of them with all loads issued before the
// stores (the pools and the rows may alias as far as the compiler knows).
template <typename T, int D, int BS, int kThreads>
__device__ __forceinline__ void append_extra_rows(const DecodeParams& prm, int first, int count) {
  constexpr int kChunks = D * static_cast<int>(sizeof(T)) / 16;  // 16-byte chunks per row
  constexpr int kBatch = kExtraChunksPerThread;
  const int row_chunks = prm.num_heads * kChunks;
  const int total = count * row_chunks;
  const char* src_k = static_cast<const char*>(prm.extra_key);
  const char* src_v = static_cast<const char*>(prm.extra_value);
  char* dst_k = static_cast<char*>(const_cast<void*>(prm.key_cache));
  char* dst_v = static_cast<char*>(const_cast<void*>(prm.value_cache));
  for (int base = threadIdx.x; base < total; base += kThreads * kBatch) {
    u32x4 kv[kBatch], vv[kBatch];
    size_t to[kBatch];
    bool live[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int idx = base + j * kThreads;
      live[j] = idx < total;
      if (!live[j]) continue;
      const int tok = first + idx / row_chunks;
      const int r = idx - (idx / row_chunks) * row_chunks;  // head * kChunks + chunk
      const int slot = prm.extra_slots[tok];
      live[j] = slot >= 0;
      if (!live[j]) continue;
      const int h = r / kChunks;
      const int c = r - h * kChunks;
      const size_t from = (static_cast<size_t>(tok) * row_chunks + r) * 16;
      to[j] = ((static_cast<size_t>(slot / BS) * prm.num_heads + h) * BS + slot % BS) * (D * sizeof(T)) +
              static_cast<size_t>(c) * 16;
      kv[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src_k + from));
      vv[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src_v + from));
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (!live[j]) continue;
      store16(dst_k + to[j], kv[j]);
      store16(dst_v + to[j], vv[j]);
    }
  }
}

// ---------------------------------------------------------------------------------
// decode, partition pass
// grid (max partitions, heads, seqs + store slices + extra slices), W wave64s
// ---------------------------------------------------------------------------------

// One workgroup of the partition pass: partition `part` of heads [HU * hg, HU * hg +
// HU) of grid slice `z` (a sequence, or one of the trailing store / append slices).
template <typename T, int D, int BS, int W, int HU>
__device__ __forceinline__ void partitions_workgroup(const DecodeParams& prm, int part, int hg, int z) {
  using G = Geometry<T, D, BS>;
  constexpr int kVec = G::kVec;
  constexpr int kThreads = kWave * W;
  const int head_groups = prm.num_heads / HU;  // grid y
  const int head = hg * HU;                    // first head of the workgroup

  if (z >= prm.num_seqs) {
    // store_slices(): one store workgroup per sequence, num_partitions * num_heads a slice
    const int64_t per_slice = static_cast<int64_t>(prm.num_partitions) * head_groups;
    const int z_extra =
        prm.num_seqs + (prm.new_key ? static_cast<int>((prm.num_seqs + per_slice - 1) / per_slice) : 0);
    if (z < z_extra) {  // pa_decode_append's store workgroups, one per sequence
      const int64_t s = (static_cast<int64_t>(z - prm.num_seqs) * head_groups + hg) *
                            prm.num_partitions + part;
      if (s < prm.num_seqs) store_new_row<T, D, BS, kThreads>(prm, static_cast<int>(s));
    } else {  // workgroups appending the extra rows, extra_per_group each
      const int64_t g = (static_cast<int64_t>(z - z_extra) * head_groups + hg) * prm.num_partitions + part;
      const int64_t first = g * prm.extra_per_group;
      if (first < prm.extra_tokens)
        append_extra_rows<T, D, BS, kThreads>(
            prm, static_cast<int>(first),
            static_cast<int>(min(static_cast<int64_t>(prm.extra_per_group), prm.extra_tokens - first)));
    }
    return;
  }
  // grid slice z decodes sequence z, or seq_order[z] when the caller ordered the launch
  const int seq = prm.seq_order ? __builtin_amdgcn_readfirstlane(prm.seq_order[z]) : z;
  const int P = prm.partition_tokens;
  const int start = prm.token_begin ? tiled_prefix(prm.token_begin[seq]) : 0;  // a multiple of BS
  const int tok_begin = start + part * P;
  const int unit_begin = tok_begin / G::kUnitTok;  // P and start are multiples of BS

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int row = lane / G::kLanesPerTok;
  const int col = lane % G::kLanesPerTok;
  const bool active = col < G::kActive;
  const int col_data = active ? col : 0;  // idle lanes of a padded row read column 0

  // Issued together, before anything waits on memory: the context length, the
  // query row and the blocks of this wave's first kWave units.  The ids are bounded
  // by the table row, not by the context (entries past the context are read but
  // never used), so the K/V stream waits on one dependent load instead of two.
  const int* table = prm.block_tables + static_cast<size_t>(seq) * prm.max_blocks_per_seq;
  const int first_unit = unit_begin + wave;
  const int blk0 = (first_unit + lane * W) / G::kUnitsPerBlock;
  const int ids0 = blk0 < prm.max_blocks_per_seq ? table[blk0] : 0;
  u32x4 q[HU];
#pragma unroll
  for (int h = 0; h < HU; ++h)
    q[h] = load16(static_cast<const T*>(prm.query) +
                  (static_cast<size_t>(seq) * prm.num_heads + head + h) * D + col_data * kVec);
  const int ctx = prm.context_lens[seq];
  T* out_row = static_cast<T*>(prm.out) + (static_cast<size_t>(seq) * prm.num_heads + head) * D;  // HU rows

  if (tok_begin >= ctx) {
    // no token after `start`: the prefix states alone, or zero (with states_only the
    // merge pass writes it)
    if (part == 0 && !prm.states_only) {
      for (int e = threadIdx.x; e < HU * D; e += kThreads) {
        const int d = e % D;
        float m = -INFINITY, l = 0.0f, o = 0.0f;
        if (start > 0) fold_prefix_states(prm, seq, head + e / D, start, d, D, m, l, o);
        out_row[e] = Lane16<T>::from_float(l > 0.0f ? o / l : 0.0f);
      }
    }
    return;
  }
  const int tok_end = min(ctx, tok_begin + P);
  // pa_decode_append: this partition ends with the newest token (position ctx - 1),
  // which is read from new_key / new_value and stored into the pools here; its unit
  // is then folded as a partly filled one (whole or not)
  NewRow<T> nr;
  nr.on = prm.new_key != nullptr && tok_end == ctx;
  const size_t new_at = (static_cast<size_t>(seq) * prm.num_heads + head) * D + col_data * kVec;
  nr.k = static_cast<const T*>(prm.new_key) + new_at;
  nr.v = static_cast<const T*>(prm.new_value) + new_at;
  const int full_end = (nr.on ? tok_end - 1 : tok_end) / G::kUnitTok;  // units folded whole
  const int unit_end = (tok_end + G::kUnitTok - 1) / G::kUnitTok;

  const size_t block_stride = static_cast<size_t>(prm.num_heads) * BS * D;  // elements
  const T* k_head = static_cast<const T*>(prm.key_cache) + static_cast<size_t>(head) * BS * D;
  const T* v_head = static_cast<const T*>(prm.value_cache) + static_cast<size_t>(head) * BS * D;
  const int lane_off = row * D + col_data * kVec;  // element offset of this lane in load 0
  const float scale_log2 = prm.scale * kLog2e;

  // This wave owns units first_unit + j * W, j < n_mine; the last of them may be
  // partly filled.
  const int n_total = unit_end - unit_begin;
  const int n_mine = n_total > wave ? (n_total - wave + W - 1) / W : 0;
  const int n_full = full_end - unit_begin > wave ? (full_end - unit_begin - wave + W - 1) / W : 0;
  const int tail_valid = tok_end - (first_unit + n_full * W) * G::kUnitTok;

  RowState<kVec> st[HU];
#pragma unroll
  for (int h = 0; h < HU; ++h) {
    st[h].m = -INFINITY;
    st[h].l = 0.0f;
#pragma unroll
    for (int j = 0; j < kVec; ++j) st[h].acc[j] = 0.0f;
  }
  attend_units<T, D, BS, W, HU>(st, q, ids0, table, first_unit, k_head, v_head, block_stride, lane_off,
                                lane, row, active, n_mine, n_full, tail_valid, scale_log2, nr);

  // merge the token rows of the wave (lanes with the same col), each head's in turn
#pragma unroll
  for (int h = 0; h < HU; ++h) {
#pragma unroll
    for (int off = G::kLanesPerTok; off < kWave; off <<= 1) {
      const float m_o = __shfl_xor(st[h].m, off);
      const float l_o = __shfl_xor(st[h].l, off);
      float acc_o[kVec];
#pragma unroll
      for (int j = 0; j < kVec; ++j) acc_o[j] = __shfl_xor(st[h].acc[j], off);
      merge_state<kVec>(st[h], m_o, l_o, acc_o);
    }
  }

  // merge the waves through LDS, in wave order
  __shared__ float s_m[HU][W];
  __shared__ float s_l[HU][W];
  __shared__ float s_o[HU][W][D];
  if (row == 0 && active) {
#pragma unroll
    for (int h = 0; h < HU; ++h) {
#pragma unroll
      for (int j = 0; j < kVec; ++j) s_o[h][wave][col * kVec + j] = st[h].acc[j];
      if (col == 0) {
        s_m[h][wave] = st[h].m;
        s_l[h][wave] = st[h].l;
      }
    }
  }
  __syncthreads();

  // one partition covers every token after `start`: finish here (merging the
  // prefix states, if any), no reduce pass needed for this sequence -- unless the
  // prefix states are written by the same launch (states_only)
  const bool single = !prm.states_only && ctx - start <= P;
  for (int e = threadIdx.x; e < HU * D; e += kThreads) {
    const int h = e / D;
    const int d = e - h * D;
    float m = s_m[h][0];
#pragma unroll
    for (int w = 1; w < W; ++w) m = fmaxf(m, s_m[h][w]);
    float l = 0.0f;
    float o = 0.0f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float f = (s_m[h][w] == -INFINITY) ? 0.0f : fast_exp2(s_m[h][w] - m);
      l = l + s_l[h][w] * f;
      o = o + s_o[h][w][d] * f;
    }
    if (single) {
      if (start > 0) fold_prefix_states(prm, seq, head + h, start, d, D, m, l, o);
      out_row[e] = Lane16<T>::from_float(o / l);
    } else {
      const size_t slot = (static_cast<size_t>(seq) * prm.num_heads + head + h) * prm.slots_per_pair +
                          prm.slot_offset + part;
      prm.ws_o[slot * D + d] = o;
      if (d == 0) {
        prm.ws_m[slot] = m;
        prm.ws_l[slot] = l;
      }
    }
  }
}

template <typename T, int D, int BS, int W, int HU>
__global__ __launch_bounds__(kWave * W) PA_OCCUPANCY void decode_partitions_kernel(DecodeParams prm) {
  // the executor learns from this word that the previous step's launches are done
  if (prm.started_flag && (blockIdx.x | blockIdx.y | blockIdx.z | threadIdx.x) == 0)
    *reinterpret_cast<volatile int32_t*>(prm.started_flag) = prm.step;
  partitions_workgroup<T, D, BS, W, HU>(prm, blockIdx.x, blockIdx.y, blockIdx.z);
}

// ---------------------------------------------------------------------------------
// decode, reduce pass: grid (heads, seqs), D threads
// ---------------------------------------------------------------------------------

template <typename T, int D>
__global__ __launch_bounds__(D) void decode_reduce_kernel(ReduceParams prm) {
  const int head = blockIdx.x;
  const int seq = blockIdx.y;
  const int ctx = prm.context_lens[seq];
  const int start = prm.prefix_lens ? tiled_prefix(prm.prefix_lens[seq]) : 0;
  const int P = prm.partition_tokens;
  const int Pp = prm.prefix_partition_tokens;
  const int np_suffix = ctx > start ? (ctx - start + P - 1) / P : 0;
  const int np_prefix = start > 0 ? (start + Pp - 1) / Pp : 0;
  if (!prm.merge_all && np_suffix <= 1) return;  // written directly by the partition pass
  const int d = threadIdx.x;
  const size_t base = (static_cast<size_t>(seq) * prm.num_heads + head) * prm.slots_per_pair;
  const size_t suffix = base + prm.prefix_slots;

  // prefix states first, then the states after the prefix, each in token order
  float m = -INFINITY;
  for (int p = 0; p < np_prefix; ++p) m = fmaxf(m, prm.ws_m[base + p]);
  for (int p = 0; p < np_suffix; ++p) m = fmaxf(m, prm.ws_m[suffix + p]);
  float l = 0.0f;
  float o = 0.0f;
  for (int p = 0; p < np_prefix; ++p) {
    const float f = fast_exp2(prm.ws_m[base + p] - m);
    l = l + prm.ws_l[base + p] * f;
    o = o + prm.ws_o[(base + p) * D + d] * f;
  }
  for (int p = 0; p < np_suffix; ++p) {
    const float f = fast_exp2(prm.ws_m[suffix + p] - m);
    l = l + prm.ws_l[suffix + p] * f;
    o = o + prm.ws_o[(suffix + p) * D + d] * f;
  }
  T* out_row = static_cast<T*>(prm.out) + (static_cast<size_t>(seq) * prm.num_heads + head) * D;
  out_row[d] = Lane16<T>::from_float(l > 0.0f ? o / l : 0.0f);  // no state: an empty context
}

// ---------------------------------------------------------------------------------
// decode, prefix pass of the shared-prefix decode (fp16): grid (prefix partitions,
// heads, groups x query tiles), kPrefixThreads threads; a query tile is 16 members
// of a group.
//
// A group is a range of sequences whose first prefix_len tokens live in the same
// physical blocks (shared by reference count).  Each shared block is read once for
// all of the group's queries, so the score and value products become small dense
// matrix products, run on the matrix cores as tiles of 16 tokens x 16 queries:
//   scores  S^T[t][g] = sum_d K[t][d] Q[g][d]   (v_mfma_f32_16x16x32_f16, A = K tile,
//           B = Q^T; lane l holds token l%16 of K and query l%16 of Q, both over the
//           same 8 dims per step: [32c + 8(l/16), +8) at step c; the K tile is read
//           as contiguous KiB runs and regrouped into this layout through LDS, so no
//           load instruction touches 16 rows of 64 bytes)
//   output  O^T[d][g] = sum_t V[t][d] P[g][t]   (v_mfma_f32_16x16x16_f16, A = V^T,
//           B = P^T)
// The matrix-core result layout puts tokens 4(l/16)..+3 of query l%16 in lane l,
// which is exactly the B operand layout of the value product, so the softmax
// weights never leave their lanes.  For the A operand of the value product the
// output dims are relabelled (row m of tile dt is dim D/16*m + dt), so that every
// lane loads its V rows as contiguous 16-byte runs.  The weights enter the value
// product as two fp16 terms (p = hi + lo, hi = fp16(p), lo = fp16(p - hi)), which
// keeps the products within fp32 rounding of the exact weights; accumulation is
// fp32 throughout.  Each (partition, head, sequence) leaves its partial softmax
// state in the workspace; the reduce pass merges it with the rest of the sequence.
// ---------------------------------------------------------------------------------

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#ifndef PA_PREFIX_PREFETCH
// 1: the prefix pass keeps the next tile's loads in flight (159 VGPRs at D 128: one
// 8-wave workgroup per CU); 0: one tile at a time (118 VGPRs: two workgroups fit a CU),
// measured 0.3-1.9 % faster over six group layouts
#define PA_PREFIX_PREFETCH 0
#endif
#ifndef PA_PREFIX_WAVES
#define PA_PREFIX_WAVES 8  // wave64s per prefix workgroup (4, 8 or 16)
#endif
constexpr int kPrefixWaves = PA_PREFIX_WAVES;
// wave states the LDS merge holds at once: half the waves park theirs, the other half
// fold them in (4 waves: all at once)
constexpr int kPrefixSlots = kPrefixWaves > 4 ? kPrefixWaves / 2 : kPrefixWaves;
constexpr int kPrefixThreads = kPrefixWaves * kWave;
static_assert(kPrefixWaves == kPrefixSlots || kPrefixWaves == 2 * kPrefixSlots, "prefix waves");

// One lane's run of kN fp16 values of a V row (kN = D / 16: 8, 10, 12, 16 or 32 bytes).
template <int kN> struct HalfRun;
template <> struct HalfRun<8> {
  u32x4 w;
  __device__ __forceinline__ void load(const _Float16* p) { w = load_kv16(p); }
  __device__ __forceinline__ _Float16 at(int i) const { return as_h2(w[i / 2])[i % 2]; }
};
template <> struct HalfRun<16> {
  u32x4 w[2];
  __device__ __forceinline__ void load(const _Float16* p) {
    w[0] = load_kv16(p);
    w[1] = load_kv16(p + 8);
  }
  __device__ __forceinline__ _Float16 at(int i) const { return as_h2(w[i / 8][(i % 8) / 2])[i % 2]; }
};
template <> struct HalfRun<6> {
  uint32_t w[3];
  __device__ __forceinline__ void load(const _Float16* p) {
    const uint32_t* u = reinterpret_cast<const uint32_t*>(p);  // 4-byte aligned: 12 bytes per lane
    w[0] = __builtin_nontemporal_load(u);
    w[1] = __builtin_nontemporal_load(u + 1);
    w[2] = __builtin_nontemporal_load(u + 2);
  }
  __device__ __forceinline__ _Float16 at(int i) const { return as_h2(w[i / 2])[i % 2]; }
};
template <> struct HalfRun<5> {
  // 10 bytes per lane, 2-byte aligned: the three aligned dwords around the run are read
  // (never past the end of the row: a run that starts on an odd half ends on its last
  // half, one that starts on an even half is followed by at least one more of the row)
  uint32_t w[3];
  int skip;  // 1 when the run starts on the second half of its first dword
  __device__ __forceinline__ void load(const _Float16* p) {
    skip = static_cast<int>((reinterpret_cast<uintptr_t>(p) >> 1) & 1);
    const uint32_t* u = reinterpret_cast<const uint32_t*>(p - skip);
    w[0] = __builtin_nontemporal_load(u);
    w[1] = __builtin_nontemporal_load(u + 1);
    w[2] = __builtin_nontemporal_load(u + 2);
  }
  // i is a constant after unrolling: both candidates are fixed register halves
  __device__ __forceinline__ _Float16 at(int i) const {
    const _Float16 here = as_h2(w[i / 2])[i % 2];
    const _Float16 next = as_h2(w[(i + 1) / 2])[(i + 1) % 2];
    return skip ? next : here;
  }
};
template <> struct HalfRun<4> {
  u32x2 w;
  __device__ __forceinline__ void load(const _Float16* p) {
    w = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  }
  __device__ __forceinline__ _Float16 at(int i) const { return as_h2(w[i / 2])[i % 2]; }
};

template <int D, int BS>
__device__ __forceinline__ void prefix_workgroup(const PrefixParams& prm, int part, int head, int zz) {
  static_assert((BS % kTile == 0 || BS == kTile / 2) && (D == 64 || D == 80 || D == 96 || D == 128 || D == 256),
                "shape");
  // a tile lies in one block (kTilesPerBlock tiles per block), or with blocks of 8 tokens
  // spans two (its first 8 token rows in block 2t of the table, the last 8 in block 2t + 1)
  constexpr int kBlocksPerTile = BS < kTile ? kTile / BS : 1;
  constexpr int kTilesPerBlock = BS < kTile ? 1 : BS / kTile;
  auto table_index = [](int tile, int k) { return kBlocksPerTile == 1 ? tile / kTilesPerBlock : 2 * tile + k; };
  // score product: step c (of kQLoads) gives lane group j the dims
  // [32c + 8j, 32c + 8j + 8) of its K row and query -- one 16-byte load each, and the
  // four lane groups of a row read 64 contiguous bytes per load instruction.  At D 80
  // the last step's dims 80-95 are zero on both sides (no load reads them), and the
  // tile's K (16 x D elements) is kQLoads loads of 512 elements, the last one partial.
  constexpr int kQLoads = (D + 31) / 32;
  constexpr bool kPartial = D % 32 != 0;
  constexpr int kDv = D / 16;         // dims per lane per V row, also value-product tiles
  auto k_elem_live = [](int e) { return !kPartial || e < kTile * D; };  // element e of a tile

  const int grp = zz / prm.query_tiles;
  const int qtile = zz % prm.query_tiles;  // first tile of 16 queries of this workgroup
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int c16 = lane % kTile;  // K row and query column of this lane
  const int j = lane / kTile;    // lane group
  auto dims_live = [j](int c) { return !kPartial || 32 * c + 8 * j < D; };  // step c, this lane

  const int s0 = prm.group_starts[grp];
  const int n_seqs = prm.group_starts[grp + 1] - s0;
  if (qtile * kTile >= n_seqs) return;  // an empty group, or a tile past its members
  const int P = prm.partition_tokens;
  const int tok_begin = part * P;
  const int tile_begin = tok_begin / kTile;
  const int* table = prm.block_tables + static_cast<size_t>(s0) * prm.max_blocks_per_seq;

  // B operand of the score product for the queries q0 .. q0 + 15: query q0 + c16,
  // dims [32c + 8j, +8) per step c
  u32x4 qv[kQLoads];
  auto load_queries = [&](int q0) {
    if (q0 + c16 < n_seqs) {
      const _Float16* qp = static_cast<const _Float16*>(prm.query) +
                           (static_cast<size_t>(s0 + q0 + c16) * prm.num_heads + head) * D + 8 * j;
#pragma unroll
      for (int i = 0; i < kQLoads; ++i) qv[i] = dims_live(i) ? load16(qp + 32 * i) : u32x4{0u, 0u, 0u, 0u};
    } else {
#pragma unroll
      for (int i = 0; i < kQLoads; ++i) qv[i] = u32x4{0u, 0u, 0u, 0u};
    }
  };
  // Issued before the prefix length is read, so that the K/V stream waits on one
  // dependent load (the group's first sequence) instead of two: the first tile of
  // queries, and the block ids of this wave's first 64 tiles, bounded by the partition
  // and the table row rather than by the prefix (entries past it are read, never used).
  load_queries(qtile * kTile);
  const int first_tile = tile_begin + wave + lane * kPrefixWaves;
  int ids_first[kBlocksPerTile];
#pragma unroll
  for (int k = 0; k < kBlocksPerTile; ++k)
    ids_first[k] = wave + lane * kPrefixWaves < P / kTile && table_index(first_tile, k) < prm.max_blocks_per_seq
                       ? table[table_index(first_tile, k)]
                       : 0;

  const int plen = tiled_prefix(prm.prefix_lens[s0]);
  if (tok_begin >= plen) return;
  const int tok_end = min(plen, tok_begin + P);  // a whole number of tiles
  const int n_tiles = (tok_end - tok_begin) / kTile;
  const int n_mine = n_tiles > wave ? (n_tiles - wave + kPrefixWaves - 1) / kPrefixWaves : 0;

  const size_t block_stride = static_cast<size_t>(prm.num_heads) * BS * D;  // elements
  const _Float16* k_head = static_cast<const _Float16*>(prm.key_cache) + static_cast<size_t>(head) * BS * D;
  const _Float16* v_head = static_cast<const _Float16*>(prm.value_cache) + static_cast<size_t>(head) * BS * D;
  const float scale_log2 = prm.scale * kLog2e;

  // Each wave's K tile, staged row by row (D + 8 elements per row: the 16 rows one
  // read instruction touches start on distinct banks); shares its space with the
  // merge buffers, which are used only after every wave has left the tile loop.
  constexpr int kKRow = D + 8;
  union PrefixLds {
    _Float16 k[kPrefixWaves][kTile * kKRow];
    struct {
      float m[kPrefixSlots][kTile];
      float l[kPrefixSlots][kTile];
      float o[kPrefixSlots][kTile][D + 1];  // +1: rows of one lane group hit distinct banks
    } merge;
  };
  __shared__ PrefixLds lds;
  auto& s_m = lds.merge.m;
  auto& s_l = lds.merge.l;
  auto& s_o = lds.merge.o;
  _Float16* s_k = lds.k[wave];

  // Tiles qtile, qtile + query_tiles, ...: with query_tiles at least the group size
  // / 16 (the usual case) one tile, every tile of the group in a workgroup of its own.
  for (int q0 = qtile * kTile; q0 < n_seqs; q0 += prm.query_tiles * kTile) {
    if (q0 != qtile * kTile) load_queries(q0);

    float m = -INFINITY;  // running max (base 2) of query c16
    float l = 0.0f;
    f32x4 acc[kDv];       // acc[dt][v] = O[c16][kDv * (4j + v) + dt]
#pragma unroll
    for (int dt = 0; dt < kDv; ++dt) acc[dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // Fold one tile (scores, online softmax, value product) into the state.
    auto fold_tile = [&](const u32x4 (&kraw)[kQLoads], const HalfRun<kDv> (&vr)[4]) {
      // kraw[c] holds elements [512c + 8 lane, +8) of the tile (row-major); regroup
      // them through this wave's LDS rows into the score product's A layout
      u32x4 kv[kQLoads];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int c = 0; c < kQLoads; ++c) {
        const int e = 512 * c + 8 * lane;
        if (k_elem_live(e)) *reinterpret_cast<u32x4*>(s_k + (e / D) * kKRow + e % D) = kraw[c];
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int c = 0; c < kQLoads; ++c)
        kv[c] = dims_live(c) ? *reinterpret_cast<const u32x4*>(s_k + c16 * kKRow + 32 * c + 8 * j)
                             : u32x4{0u, 0u, 0u, 0u};
      // scores: sc[v] = <K row 4j+v, query c16>
      f32x4 sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int c = 0; c < kQLoads; ++c)
        sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, kv[c]),
                                                    __builtin_bit_cast(f16x8, qv[c]), sc, 0, 0, 0);
      // online softmax of query c16 over the tile's 16 tokens (4 per lane group)
      float z[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) z[v] = sc[v] * scale_log2;
      float top = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
      top = fmaxf(top, __shfl_xor(top, 16));
      top = fmaxf(top, __shfl_xor(top, 32));
      const float m_new = fmaxf(m, top);
      const float alpha = fast_exp2(m - m_new);  // 0 before the first tile
      float p[4];
      float psum = 0.0f;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        p[v] = fast_exp2(z[v] - m_new);
        psum += p[v];
      }
      psum += __shfl_xor(psum, 16);
      psum += __shfl_xor(psum, 32);
      l = l * alpha + psum;
      m = m_new;
      if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int dt = 0; dt < kDv; ++dt) acc[dt] *= alpha;
      }
      // value product: B = P^T (token 4j+v, query c16) as hi + lo fp16 terms
      f16x4 p_hi, p_lo;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        p_hi[v] = static_cast<_Float16>(p[v]);
        p_lo[v] = static_cast<_Float16>(p[v] - static_cast<float>(p_hi[v]));
      }
#pragma unroll
      for (int dt = 0; dt < kDv; ++dt) {
        const f16x4 a = {vr[0].at(dt), vr[1].at(dt), vr[2].at(dt), vr[3].at(dt)};
        acc[dt] = __builtin_amdgcn_mfma_f32_16x16x16f16(a, p_hi, acc[dt], 0, 0, 0);
        acc[dt] = __builtin_amdgcn_mfma_f32_16x16x16f16(a, p_lo, acc[dt], 0, 0, 0);
      }
    };

    for (int base = 0; base < n_mine; base += kWave) {
      // physical block(s) of each of this wave's tiles, one tile per lane
      const int idx = base + lane;
      int ids[kBlocksPerTile];
#pragma unroll
      for (int k = 0; k < kBlocksPerTile; ++k)
        ids[k] = base == 0      ? ids_first[k]
                 : idx < n_mine ? table[table_index(tile_begin + wave + idx * kPrefixWaves, k)]
                                : 0;
      const int n_here = min(n_mine - base, kWave);
      // the wave's i-th tile of this chunk: K as 16-byte runs of the row-major tile,
      // one contiguous KiB per load instruction (regrouped through LDS when folded),
      // and V rows 4j+v (dims [kDv*c16, +kDv))
      auto load_tile = [&](int i, u32x4 (&kv)[kQLoads], HalfRun<kDv> (&vr)[4]) {
        const int tile = tile_begin + wave + (base + i) * kPrefixWaves;
        if constexpr (kBlocksPerTile == 1) {
          const int phys = __builtin_amdgcn_readlane(ids[0], i);
          const size_t off = static_cast<size_t>(phys) * block_stride +
                             static_cast<size_t>(tile % kTilesPerBlock) * kTile * D;
#pragma unroll
          for (int ii = 0; ii < kQLoads; ++ii) {
            const int e = 512 * ii + 8 * lane;
            kv[ii] = k_elem_live(e) ? load_kv16(k_head + off + e) : u32x4{0u, 0u, 0u, 0u};
          }
#pragma unroll
          for (int v = 0; v < 4; ++v) vr[v].load(v_head + off + (4 * j + v) * D + kDv * c16);
        } else {
          // token rows 0-7 from the first block, 8-15 from the second: element e of
          // the row-major tile lies in the second block from e = 8 * D on (a load may
          // straddle that boundary between lanes, never within a lane's 8 elements)
          const size_t off0 = static_cast<size_t>(__builtin_amdgcn_readlane(ids[0], i)) * block_stride;
          const size_t off1 = static_cast<size_t>(__builtin_amdgcn_readlane(ids[1], i)) * block_stride;
#pragma unroll
          for (int ii = 0; ii < kQLoads; ++ii) {
            const int e = 512 * ii + 8 * lane;
            kv[ii] = !k_elem_live(e) ? u32x4{0u, 0u, 0u, 0u}
                     : e < 8 * D     ? load_kv16(k_head + off0 + e)
                                     : load_kv16(k_head + off1 + (e - 8 * D));
          }
          const size_t off_v = j < 2 ? off0 : off1;  // rows 4j .. 4j + 3
#pragma unroll
          for (int v = 0; v < 4; ++v) vr[v].load(v_head + off_v + (4 * (j % 2) + v) * D + kDv * c16);
        }
      };
#if PA_PREFIX_PREFETCH
      // two tiles in registers: the next tile's loads are in flight while the
      // current one is folded
      u32x4 ka[kQLoads], kb[kQLoads];
      HalfRun<kDv> va[4], vb[4];
      int i = 0;
      load_tile(0, ka, va);
      for (; i + 1 < n_here; i += 2) {
        load_tile(i + 1, kb, vb);
        fold_tile(ka, va);
        if (i + 2 < n_here) load_tile(i + 2, ka, va);
        fold_tile(kb, vb);
      }
      if (i < n_here) fold_tile(ka, va);
#else
      for (int i = 0; i < n_here; ++i) {
        u32x4 kv[kQLoads];
        HalfRun<kDv> vr[4];
        load_tile(i, kv, vr);
        fold_tile(kv, vr);
      }
#endif
    }

    // Merge the waves and leave one state per (sequence, head, partition).  The LDS
    // holds kPrefixSlots wave states: with more waves than slots, the upper waves
    // park theirs first and the lower ones fold them in, in a fixed order.
    auto park = [&](int slot) {
      if (j == 0) {
        s_m[slot][c16] = m;
        s_l[slot][c16] = l;
      }
#pragma unroll
      for (int dt = 0; dt < kDv; ++dt) {
#pragma unroll
        for (int v = 0; v < 4; ++v) s_o[slot][c16][kDv * (4 * j + v) + dt] = acc[dt][v];
      }
    };
    __syncthreads();  // every wave is done with its K rows before the merge reuses them
    if constexpr (kPrefixWaves > kPrefixSlots) {
      if (wave >= kPrefixSlots) park(wave - kPrefixSlots);
      __syncthreads();
      if (wave < kPrefixSlots) {
        const float m_b = s_m[wave][c16];
        const float mm = fmaxf(m, m_b);
        const float fa = (m == -INFINITY) ? 0.0f : fast_exp2(m - mm);
        const float fb = (m_b == -INFINITY) ? 0.0f : fast_exp2(m_b - mm);
        l = l * fa + s_l[wave][c16] * fb;
#pragma unroll
        for (int dt = 0; dt < kDv; ++dt) {
#pragma unroll
          for (int v = 0; v < 4; ++v)
            acc[dt][v] = acc[dt][v] * fa + s_o[wave][c16][kDv * (4 * j + v) + dt] * fb;
        }
        m = mm;
      }
      __syncthreads();
    }
    if (wave < kPrefixSlots) park(wave);
    __syncthreads();
    for (int e = threadIdx.x; e < kTile * D; e += kPrefixThreads) {
      const int g = e / D;
      const int d = e % D;
      if (q0 + g >= n_seqs) break;  // e grows with g
      float mm = s_m[0][g];
#pragma unroll
      for (int w = 1; w < kPrefixSlots; ++w) mm = fmaxf(mm, s_m[w][g]);
      float ll = 0.0f;
      float oo = 0.0f;
#pragma unroll
      for (int w = 0; w < kPrefixSlots; ++w) {
        const float f = (s_m[w][g] == -INFINITY) ? 0.0f : fast_exp2(s_m[w][g] - mm);
        ll = ll + s_l[w][g] * f;
        oo = oo + s_o[w][g][d] * f;
      }
      const size_t slot = (static_cast<size_t>(s0 + q0 + g) * prm.num_heads + head) * prm.slots_per_pair + part;
      prm.ws_o[slot * D + d] = oo;
      if (d == 0) {
        prm.ws_m[slot] = mm;
        prm.ws_l[slot] = ll;
      }
    }
    __syncthreads();  // the LDS arrays are reused by the next tile of queries
  }
}

template <int D, int BS>
__global__ __launch_bounds__(kPrefixThreads) void decode_prefix_kernel(PrefixParams prm) {
  prefix_workgroup<D, BS>(prm, blockIdx.x, blockIdx.y, blockIdx.z);
}

#if PA_SHARED_FUSED
// ---------------------------------------------------------------------------------
// shared-prefix decode in one launch: the prefix pass's workgroups first, then the
// pass over each sequence's tokens after its prefix, which writes partial states
// (DecodeParams::states_only) for the merge pass; 1-D grid, kPrefixThreads threads.
// The prefix workgroups of a batch are few (one per group, query tile, head and
// prefix partition); launched alone they leave most of the chip's wave slots idle,
// here the other pass fills them.
// ---------------------------------------------------------------------------------

template <int D, int BS>
__global__ __launch_bounds__(kPrefixThreads) void decode_shared_fused_kernel(PrefixParams pp, DecodeParams dp,
                                                                            int32_t prefix_groups) {
  static_assert(kPrefixThreads == kWave * kDecodeWavesNarrow, "one workgroup size for both passes");
  const int i = blockIdx.x;
  if (i < prefix_groups) {
    const int np = pp.num_partitions;
    const int h = pp.num_heads;
    prefix_workgroup<D, BS>(pp, i % np, (i / np) % h, i / (np * h));
  } else {
    const int j = i - prefix_groups;
    const int np = dp.num_partitions;
    const int h = dp.num_heads;
    partitions_workgroup<_Float16, D, BS, kDecodeWavesNarrow, 1>(dp, j % np, (j / np) % h, j / (np * h));
  }
}
#endif  // PA_SHARED_FUSED

// ---------------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------------

// z-slices of store workgroups pa_decode_append adds: one workgroup per sequence,
// num_partitions * (num_heads / heads_per_unit) of them per slice
int32_t store_slices(const DecodeParams& prm) {
  if (!prm.new_key || prm.num_seqs == 0) return 0;
  const int64_t per_slice = static_cast<int64_t>(prm.num_partitions) * (prm.num_heads / prm.heads_per_unit);
  return static_cast<int32_t>((prm.num_seqs + per_slice - 1) / per_slice);
}

// z-slices of the workgroups appending extra rows, extra_per_group rows each
int32_t extra_slices(const DecodeParams& prm) {
  if (!prm.extra_key || prm.extra_tokens <= 0 || prm.extra_per_group <= 0) return 0;
  const int64_t groups = (static_cast<int64_t>(prm.extra_tokens) + prm.extra_per_group - 1) / prm.extra_per_group;
  const int64_t per_slice = static_cast<int64_t>(prm.num_partitions) * (prm.num_heads / prm.heads_per_unit);
  return static_cast<int32_t>((groups + per_slice - 1) / per_slice);
}

template <typename T, int D, int BS, int HU>
static void launch_partitions_h(const DecodeParams& prm, hipStream_t stream) {
  // pa_decode_append adds z-slices after the last sequence: one workgroup per sequence
  // stores its new rows; the executor's extra rows follow
  dim3 grid(prm.num_partitions, prm.num_heads / HU, prm.num_seqs + store_slices(prm) + extra_slices(prm));
  if (prm.wide) {
    hipLaunchKernelGGL((decode_partitions_kernel<T, D, BS, kWavesWide, HU>), grid, dim3(kWave * kWavesWide), 0,
                       stream, prm);
  } else {
    hipLaunchKernelGGL((decode_partitions_kernel<T, D, BS, kWavesNarrow, HU>), grid, dim3(kWave * kWavesNarrow), 0,
                       stream, prm);
  }
}

template <typename T, int D, int BS>
static hipError_t launch_partitions_t(const DecodeParams& prm, hipStream_t stream) {
  constexpr int kMaxHU = Geometry<T, D, BS>::kMaxHeadsPerUnit;
  if (prm.heads_per_unit != 1 && prm.heads_per_unit != kMaxHU) return hipErrorInvalidValue;
  if constexpr (kMaxHU > 1) {
    if (prm.heads_per_unit == kMaxHU) {
      launch_partitions_h<T, D, BS, kMaxHU>(prm, stream);
      return hipGetLastError();
    }
  }
  launch_partitions_h<T, D, BS, 1>(prm, stream);
  return hipGetLastError();
}

template <typename T, int D>
static int32_t heads_per_unit_d(int block_size) {
  switch (block_size) {
    case 8: return Geometry<T, D, 8>::kMaxHeadsPerUnit;
    case 16: return Geometry<T, D, 16>::kMaxHeadsPerUnit;
    case 32: return Geometry<T, D, 32>::kMaxHeadsPerUnit;
    case 64: return Geometry<T, D, 64>::kMaxHeadsPerUnit;
    case 128: return Geometry<T, D, 128>::kMaxHeadsPerUnit;
    case 256: return Geometry<T, D, 256>::kMaxHeadsPerUnit;
    default: return 1;
  }
}

template <typename T>
static int32_t heads_per_unit_t(int head_dim, int block_size) {
  switch (head_dim) {
    case 64: return heads_per_unit_d<T, 64>(block_size);
    case 80: return heads_per_unit_d<T, 80>(block_size);
    case 96: return heads_per_unit_d<T, 96>(block_size);
    case 128: return heads_per_unit_d<T, 128>(block_size);
    case 256: return heads_per_unit_d<T, 256>(block_size);
    default: return 1;
  }
}

int32_t decode_heads_per_unit(bool f16, int head_dim, int block_size, int num_heads) {
  const int32_t hu = f16 ? heads_per_unit_t<_Float16>(head_dim, block_size) : heads_per_unit_t<float>(head_dim, block_size);
  return (hu > 1 && num_heads % hu == 0) ? hu : 1;
}

template <typename T, int D>
static hipError_t launch_partitions_d(const DecodeParams& prm, int block_size, hipStream_t stream) {
  switch (block_size) {
    case 8: return launch_partitions_t<T, D, 8>(prm, stream);
    case 16: return launch_partitions_t<T, D, 16>(prm, stream);
    case 32: return launch_partitions_t<T, D, 32>(prm, stream);
    case 64: return launch_partitions_t<T, D, 64>(prm, stream);
    case 128: return launch_partitions_t<T, D, 128>(prm, stream);
    case 256: return launch_partitions_t<T, D, 256>(prm, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
static hipError_t launch_partitions_dt(const DecodeParams& prm, int head_dim, int block_size,
                                       hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_partitions_d<T, 64>(prm, block_size, stream);
    case 80: return launch_partitions_d<T, 80>(prm, block_size, stream);
    case 96: return launch_partitions_d<T, 96>(prm, block_size, stream);
    case 128: return launch_partitions_d<T, 128>(prm, block_size, stream);
    case 256: return launch_partitions_d<T, 256>(prm, block_size, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_partitions(const DecodeParams& prm, bool f16, int head_dim,
                                    int block_size, hipStream_t stream) {
  return f16 ? launch_partitions_dt<_Float16>(prm, head_dim, block_size, stream)
             : launch_partitions_dt<float>(prm, head_dim, block_size, stream);
}

template <typename T, int D>
static void launch_reduce_td(const ReduceParams& prm, hipStream_t stream) {
  dim3 grid(prm.num_heads, prm.num_seqs);
  hipLaunchKernelGGL((decode_reduce_kernel<T, D>), grid, dim3(D), 0, stream, prm);
}

template <typename T>
static hipError_t launch_reduce_t(const ReduceParams& prm, int head_dim, hipStream_t stream) {
  switch (head_dim) {
    case 64: launch_reduce_td<T, 64>(prm, stream); break;
    case 80: launch_reduce_td<T, 80>(prm, stream); break;
    case 96: launch_reduce_td<T, 96>(prm, stream); break;
    case 128: launch_reduce_td<T, 128>(prm, stream); break;
    case 256: launch_reduce_td<T, 256>(prm, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_reduce(const ReduceParams& prm, bool f16, int head_dim, hipStream_t stream) {
  return f16 ? launch_reduce_t<_Float16>(prm, head_dim, stream)
             : launch_reduce_t<float>(prm, head_dim, stream);
}

template <int D>
static hipError_t launch_prefix_d(const PrefixParams& prm, int block_size, hipStream_t stream) {
  dim3 grid(prm.num_partitions, prm.num_heads, prm.num_groups * prm.query_tiles);
  switch (block_size) {
    case 8:
      hipLaunchKernelGGL((decode_prefix_kernel<D, 8>), grid, dim3(kPrefixThreads), 0, stream, prm);
      break;
    case 16:
      hipLaunchKernelGGL((decode_prefix_kernel<D, 16>), grid, dim3(kPrefixThreads), 0, stream, prm);
      break;
    case 32:
      hipLaunchKernelGGL((decode_prefix_kernel<D, 32>), grid, dim3(kPrefixThreads), 0, stream, prm);
      break;
    case 64:
      hipLaunchKernelGGL((decode_prefix_kernel<D, 64>), grid, dim3(kPrefixThreads), 0, stream, prm);
      break;
    case 128:
      hipLaunchKernelGGL((decode_prefix_kernel<D, 128>), grid, dim3(kPrefixThreads), 0, stream, prm);
      break;
    case 256:
      hipLaunchKernelGGL((decode_prefix_kernel<D, 256>), grid, dim3(kPrefixThreads), 0, stream, prm);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

#if PA_SHARED_FUSED
template <int D>
static hipError_t launch_fused_d(const PrefixParams& pp, const DecodeParams& dp, int block_size,
                                 hipStream_t stream) {
  const int64_t prefix_groups =
      static_cast<int64_t>(pp.num_partitions) * pp.num_heads * pp.num_groups * pp.query_tiles;
  const int64_t groups = prefix_groups + static_cast<int64_t>(dp.num_partitions) * dp.num_heads * dp.num_seqs;
  const dim3 grid(static_cast<unsigned>(groups));
  const int32_t pg = static_cast<int32_t>(prefix_groups);
  switch (block_size) {
    case 8: hipLaunchKernelGGL((decode_shared_fused_kernel<D, 8>), grid, dim3(kPrefixThreads), 0, stream, pp, dp, pg); break;
    case 16: hipLaunchKernelGGL((decode_shared_fused_kernel<D, 16>), grid, dim3(kPrefixThreads), 0, stream, pp, dp, pg); break;
    case 32: hipLaunchKernelGGL((decode_shared_fused_kernel<D, 32>), grid, dim3(kPrefixThreads), 0, stream, pp, dp, pg); break;
    case 64: hipLaunchKernelGGL((decode_shared_fused_kernel<D, 64>), grid, dim3(kPrefixThreads), 0, stream, pp, dp, pg); break;
    case 128: hipLaunchKernelGGL((decode_shared_fused_kernel<D, 128>), grid, dim3(kPrefixThreads), 0, stream, pp, dp, pg); break;
    case 256: hipLaunchKernelGGL((decode_shared_fused_kernel<D, 256>), grid, dim3(kPrefixThreads), 0, stream, pp, dp, pg); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_shared_fused(const PrefixParams& pp, const DecodeParams& dp, int head_dim, int block_size,
                                      hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_fused_d<64>(pp, dp, block_size, stream);
    case 80: return launch_fused_d<80>(pp, dp, block_size, stream);
    case 96: return launch_fused_d<96>(pp, dp, block_size, stream);
    case 128: return launch_fused_d<128>(pp, dp, block_size, stream);
    case 256: return launch_fused_d<256>(pp, dp, block_size, stream);
    default: return hipErrorInvalidValue;
  }
}
#endif  // PA_SHARED_FUSED

hipError_t launch_decode_prefix(const PrefixParams& prm, int head_dim, int block_size,
                                hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_prefix_d<64>(prm, block_size, stream);
    case 80: return launch_prefix_d<80>(prm, block_size, stream);
    case 96: return launch_prefix_d<96>(prm, block_size, stream);
    case 128: return launch_prefix_d<128>(prm, block_size, stream);
    case 256: return launch_prefix_d<256>(prm, block_size, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
