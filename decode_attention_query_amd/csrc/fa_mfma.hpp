// fa_mfma.hpp -- the matrix-core (MFMA) decode kernel for f32 / f16 / bf16 K/V
// on gfx950.
//
// One workgroup = one split unit of one KV head and a block of up to 16 query
// heads of its group (the whole group when G <= 16, any G), so K and V are
// read from HBM once for all those heads.  Four waves (two at D = 256); each wave
// streams its own tiles of the unit (32 rows for 16-bit K/V, 16 for f32),
// loads whole rows from HBM, stages K and V in its LDS area, and keeps its own
// online-softmax state; the waves are merged through LDS at the end.  A group
// of more than 16 heads is cut into blocks of 16 (the last one shorter, or
// empty) and takes two blocks per workgroup: every wave computes each of its
// tiles for both blocks (NB = 2 below).
//
// Per 32-row 16-bit tile, with n = lane % 16 and grp = lane / 16:
//   scores   S^T[t][g] = sum_d K[t][d] Q[g][d]        v_mfma_f32_16x16x32 (bf16|f16)
//            A = K rows read back from LDS (lane: row n of a 16-row block, 8
//            features at 32kk + 8grp), B = Q^T (lane: head n, in registers).
//            Result: lane holds S for head g = n and rows 4grp + i (i < 4) of
//            each of the two 16-row blocks.
//   softmax  per head (column): the tile max over the 32 rows (in-lane max of
//            8, then across the four lane groups), one rescale of the running
//            state, p = 2^(s - m).
//   P.V      O^T[d][g] += sum_t V[t][d] P[t][g]      v_mfma_f32_16x16x32
//            B = P^T is exactly the lane's 8 probabilities (row order below),
//            A = V^T is read from the wave's LDS copy of its V tile with
//            ds_read_b64_tr_b16: in each 16-lane group, lane 4r + b names row r,
//            features 4b .. 4b + 3 of a 4 x 16 block and lane L receives column
//            L, i.e. 4 rows of one feature -- half an A operand per read.
//            bf16 P keeps 8 bits, so P is split into hi + lo bf16 parts (two
//            MFMAs) to keep P.V at ~16-bit accuracy; f16 P is used as is.
// The contraction index k of both P.V operands is mapped to tile rows as
// row(k = 8 grp + i) = 16 (i / 4) + 4 grp + (i % 4), which is where the score
// MFMA left each lane's probabilities; any k order works as long as A and B
// agree, which they do by construction.
//
// f32 tiles (16 rows) use v_mfma_f32_16x16x4_f32, one element per lane and
// operand: the scores split D into four quarters, lane group grp taking
// features grp D/4 .. + D/4 in successive products; P.V takes four rows per
// product, lane group grp contributing row 4grp + i, so B is the lane's own
// probability and A one f32 of V read from LDS.
#pragma once

#include "fa_common.hpp"
#include "fa_kernels.hpp"

namespace fa {

template <class E>
struct Mfma;

template <>
struct Mfma<BF16> {
  typedef __bf16 v8 __attribute__((ext_vector_type(8)));
  typedef __bf16 v2 __attribute__((ext_vector_type(2)));
  static constexpr bool kSplitP = true;
  __device__ static inline f32x4 mma(v8 a, v8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Mfma<F16> {
  typedef _Float16 v8 __attribute__((ext_vector_type(8)));
  typedef _Float16 v2 __attribute__((ext_vector_type(2)));
  static constexpr bool kSplitP = false;
  __device__ static inline f32x4 mma(v8 a, v8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

// f32 K/V: v_mfma_f32_16x16x4_f32, one element per lane and operand (A: lane
// l holds A[l % 16][l / 16]; B: B[l / 16][l % 16]; the 16x16 result in the
// same lane layout as the 16-bit products).  v8 is unused on this path.
template <>
struct Mfma<F32> {
  typedef float v8 __attribute__((ext_vector_type(8)));
  static constexpr bool kSplitP = false;
  __device__ static inline f32x4 mma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

// 8 probabilities -> MFMA operand(s), round-to-nearest-even; with kSplitP the
// residual p - hi is rounded into lo, so hi + lo carries ~16 significant bits.
template <class E>
__device__ inline void pack_probs(const float *p, typename Mfma<E>::v8 &hi,
                                  typename Mfma<E>::v8 &lo) {
  using M = Mfma<E>;
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    const f32x2 f = {p[e], p[e + 1]};
    const typename M::v2 h = __builtin_convertvector(f, typename M::v2);
    hi[e] = h[0];
    hi[e + 1] = h[1];
    if constexpr (M::kSplitP) {
      const f32x2 back = __builtin_convertvector(h, f32x2);
      const f32x2 r = {f[0] - back[0], f[1] - back[1]};
      const typename M::v2 l = __builtin_convertvector(r, typename M::v2);
      lo[e] = l[0];
      lo[e + 1] = l[1];
    }
  }
}


// Waves per workgroup: four, but two at D = 256, whose K/V tiles would fill
// 137 KB of LDS at four waves; at two, two workgroups share a compute unit, so
// one streams while the other starts or finishes.
constexpr int mfma_waves(int d) { return d <= 128 ? 4 : 2; }

template <class E, int D>
struct MfmaGeom {
  static constexpr bool kF32 = E::kBytes == 4;
  static constexpr int NW = mfma_waves(D);
  // rows per wave tile: 32 (two 16-row MFMA blocks) for 16-bit K/V; 16 for
  // f32, whose rows are twice as wide (the same 16 KiB per tile at D = 128)
  static constexpr int TT = kF32 ? 16 : 32;
  static constexpr int JB = TT / 16;     // 16-row blocks per tile
  static constexpr int KK = D / 32;      // 16-bit score k-steps (k = 32) per 16-row block
  static constexpr int QC = D / 16;      // f32: 4-feature chunks of a lane's quarter of D
  static constexpr int MB = D / 16;      // 16-feature blocks of O^T
  // Global loads: each instruction reads whole rows, 1 KiB contiguous per
  // wave (LPR lanes per row, RPI rows per instruction, NI instructions per
  // tile of K, and as many of V).  An instruction shaped like the MFMA
  // operand instead (16 rows x 64 bytes) streams ~13% slower from HBM.
  static constexpr int LPR = D * E::kBytes / 16;
  static constexpr int RPI = 64 / LPR;
  static constexpr int NI = TT / RPI;
  // LDS row strides.  K is read back 16 bytes per lane from 16 rows at once:
  // a 16-byte pad puts those rows in distinct banks.  16-bit V is read with
  // transposed 8-byte reads spanning 8 rows: a 32-byte pad does the same; f32
  // V is read 4 bytes per lane, 16 features of 4 rows at once: a 64-byte pad
  // puts the 4 rows in distinct banks.
  static constexpr int ROWK = D * E::kBytes + 16;
  static constexpr int ROWV = kF32 ? D * 4 + 64 : D * 2 + 32;
  static constexpr int WAVE_LDS = TT * (ROWK + ROWV);
  static constexpr int LDS_KV = NW * WAVE_LDS;
  // Wave-merge area (reuses the K/V area): per wave 16 head rows of D floats,
  // padded by 16 bytes so that the 16 lanes writing one feature block of 16
  // different heads hit distinct banks (an unpadded 2^k-byte row puts them
  // all in one).
  static constexpr int ACC_ROW = D + 4;
  static constexpr int LDS_ACC = NW * 16 * ACC_ROW * 4;
  static constexpr int LDS = LDS_KV > LDS_ACC ? LDS_KV : LDS_ACC;
  // two register tiles, ping-pong (D <= 128); at D = 256 one, reloaded as
  // soon as it is in LDS
  static constexpr bool kPipelined = D <= 128;
};

// The page ids of the unit's rows [t_begin, t_end), once, into LDS
// (s_pages[i] = page id of page slot slot0 + i, clamped into the pool), so
// that each tile's lookups are LDS reads instead of memory loads it would wait
// for; returns slot0.  Only when every 16-row block lies in one page (else
// issue_tile resolves rows itself).  The host keeps a unit within kPageTable
// page slots.  Every thread of the workgroup calls it (it ends in a barrier).
__device__ inline int stage_unit_pages(const DecodeParams &p, int32_t *s_pages,
                                       int32_t page_base, int t_begin, int t_end,
                                       int nthreads) {
  int slot0 = 0;
  if (p.uniform_blocks && !p.contig && t_begin < t_end) {
    slot0 = (int)fastdiv((uint32_t)t_begin, p.page_div);
    const int count = (int)fastdiv((uint32_t)(t_end - 1), p.page_div) - slot0 + 1;
    for (int i = threadIdx.x; i < count; i += nthreads) {
      const int32_t id = p.indices[page_base + slot0 + i];
      s_pages[i] = min(max(id, 0), p.num_total_pages - 1);
    }
    __syncthreads();
  }
  return slot0;
}

// K and V of one tile as loaded: instruction i, lane l holds row
// RPI * i + l / LPR, bytes 16 (l % LPR) .. + 16.
template <int NI>
struct KVTile {
  uint4 k[NI];
  uint4 v[NI];
};

// Element offset of the first row of the 16-row block starting at row tb
// (wave-uniform; the block lies in one page).  Page ids come from the unit's
// slice of the page table, staged in LDS at the start of the workgroup
// (s_pages[i] = page id of page slot slot0 + i).
template <bool kNhd>
__device__ inline int64_t staged_block_offset(const DecodeParams &p, const int32_t *s_pages,
                                              int slot0, int kvh, int tb) {
  int64_t page = 0;
  uint32_t row = (uint32_t)tb;
  if (!p.contig) {
    const uint32_t slot = fastdiv((uint32_t)tb, p.page_div);
    row = (uint32_t)tb - slot * (uint32_t)p.page_size;
    page = __builtin_amdgcn_readfirstlane(s_pages[slot - slot0]);
  }
  return kv_elem_offset<kNhd>(p, page, kvh, row);
}

// Issues the global loads of the tile whose first row is t0 (rows past t_end
// are clamped to t_end - 1: in bounds, and masked out of the softmax later).
// t0, t_end and page_base are wave-uniform.  When every 16-row block lies in
// one page, the block's page comes from LDS once per block and rows follow at
// the layout's row stride (D heads-major, Hkv * D token-major); otherwise
// (page sizes that are not multiples of 16) every lane resolves its own rows.
template <class E, int D, bool kNhd>
__device__ __forceinline__ void issue_tile(KVTile<MfmaGeom<E, D>::NI> &T, const DecodeParams &p,
                                  int32_t page_base, const int32_t *s_pages, int slot0, int kvh,
                                  int t0, int t_end, int lane) {
  using G = MfmaGeom<E, D>;
  const int64_t rs = kNhd ? (int64_t)p.num_kv_heads * D : D;  // elements between rows
  const int r0 = lane / G::LPR;           // row within an instruction
  const int col = (lane % G::LPR) * 16;   // byte within the row
  const char *kb = static_cast<const char *>(p.k) + col;
  const char *vb = static_cast<const char *>(p.v) + col;
  int64_t blk[G::JB];
  if (p.uniform_blocks) {
#pragma unroll
    for (int j = 0; j < G::JB; ++j) {
      const int tb = min(t0 + 16 * j, t_end - 1);
      blk[j] = staged_block_offset<kNhd>(p, s_pages, slot0, kvh, tb) - (int64_t)tb * rs;
    }
  }
#pragma unroll
  for (int i = 0; i < G::NI; ++i) {
    const int r = G::RPI * i + r0;  // row within the tile
    const int t = min(t0 + r, t_end - 1);
    int64_t off;
    if (p.uniform_blocks) {
      // rows of block j = r / 16 share its page: offset = block base + row stride
      off = (blk[(G::RPI * i) / 16] + (int64_t)t * rs) * E::kBytes;
    } else {
      off = kv_row_offset(p, page_base, kvh, t) * E::kBytes;
    }
    T.k[i] = load16_stream(kb + off);
    T.v[i] = load16_stream(vb + off);
  }
}

// kMods: a sliding window, soft-cap, ALiBi or custom mask is in use (the
// plain instance carries none of their per-score work, nor the mask's tile
// lookups).
//
// NB: 16-column head blocks per workgroup.  NB = 1: the workgroup's one block
// (the whole group when G <= 16).  NB = 2 (a query group of more than 16
// heads, e.g. G = 32), D <= 128: every wave computes each tile it loads for
// both blocks -- one K operand read from LDS feeds both blocks' score
// products and one V^T read both blocks' P.V products -- so K and V leave HBM
// once for 32 query heads and the waves stream independently, with no
// workgroup barrier inside the main loop.  The second block's query operands,
// accumulators and softmax state take the registers of the second K/V tile,
// so one register tile is in flight while the other is computed (the D = 256
// loop).  NB = 2 where a wave's registers do not hold two blocks' state
// beside a tile (D = 256; f32 at D = 128 with the per-score options): the
// waves share each step's tiles through LDS instead, and after a workgroup
// barrier the first half of the waves computes every tile of the step for
// block 0 and the second half for block 1.
template <class E, int D, bool kNhd, bool kMods, int NB>
__global__ __launch_bounds__(mfma_waves(D) * 64) __attribute__((amdgpu_waves_per_eu(D <= 128 ? 2 : 1))) void decode_mfma_kernel(
    const DecodeParams p) {
  using G = MfmaGeom<E, D>;
  using M = Mfma<E>;
  using v8 = typename M::v8;
  constexpr int KK = G::KK, MB = G::MB, NW = G::NW, TT = G::TT, JB = G::JB, QC = G::QC;
  constexpr bool kF32 = G::kF32;
  static_assert(NB == 1 || NB == 2, "head blocks per workgroup");
  // head blocks per wave (NBW), and whether the waves share tiles (kShared:
  // wave w serves block w / WPB of the workgroup's NB) -- where two blocks'
  // state does not fit a wave's registers beside a tile: D = 256, and f32 at
  // D = 128 with the per-score options
  constexpr bool kShared = NB == 2 && (D > 128 || (kF32 && D == 128 && kMods));
  constexpr int NBW = kShared ? 1 : NB;
  constexpr int WPB = kShared ? NW / NB : NW;
  static_assert(!kShared || NW % NB == 0, "waves per head block");
  // two register tiles in flight only where the registers allow it
  constexpr bool kPipe = G::kPipelined && NBW == 1;
  // the wave-merge area (per wave NBW * 16 head rows) fits the K/V area
  static_assert(NW * 16 * NBW * G::ACC_ROW * 4 <= G::LDS, "wave-merge area");

  __shared__ __attribute__((aligned(16))) char lds[G::LDS];
  __shared__ float s_m[NW][16 * NBW];
  __shared__ float s_l[NW][16 * NBW];
  __shared__ float s_stat[2 * kStatHeads];
  __shared__ int s_last;
  __shared__ int s_work;
  __shared__ uint32_t s_mask[NW];  // shared tiles: each wave's tile mask word

  // work item = unit * planes + head block: a unit's head blocks are adjacent,
  // and work items run in (longest-first) unit order.  The first resident
  // round takes its item from its launch index; later workgroups draw theirs.
  int w = blockIdx.x;
  if (w >= p.ticket_from) {
    if (threadIdx.x == 0)
      s_work = p.ticket_from + draw_ticket(reinterpret_cast<unsigned long long *>(p.tickets),
                                           (int)gridDim.x - p.ticket_from);
    __syncthreads();
    w = __builtin_amdgcn_readfirstlane(s_work);
  }
  const int unit = w / p.planes;
  const int plane = w - unit * p.planes;
  UnitInfo u;
  if (!find_unit<kMods>(p, unit, u)) return;  // row0 (for a custom mask) in the kMods instance
  // Head blocks of bs = heads_per_unit query heads (the whole group when it
  // has at most 16, else 16 with a shorter last block); the workgroup serves
  // blocks NB * gblock .. + NB - 1 of its KV head's group, gt_wg heads in all.
  const int bs = p.heads_per_unit;
  const int kvh = plane / p.n_gblocks;
  const int gblock = plane - kvh * p.n_gblocks;
  const int h0 = kvh * p.group + gblock * NB * bs;  // the workgroup's first head
  const int gt_wg = min(NB * bs, p.group - gblock * NB * bs);
  // workgroup-uniform values, kept in scalar registers
  const int t_begin = __builtin_amdgcn_readfirstlane(u.lo + u.c * p.chunk);
  const int t_end = __builtin_amdgcn_readfirstlane(min(u.L, t_begin + p.chunk));
  const int t_lo = __builtin_amdgcn_readfirstlane(u.start);  // rows below: outside the window
  const int last_row = __builtin_amdgcn_readfirstlane(u.L - 1);
  const int32_t page_base = __builtin_amdgcn_readfirstlane(u.page_base);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;
  const int grp = lane >> 4;
  // the wave's k-th block (block wb0 + k of the workgroup): first head hb[k]
  // (past the group when the block is empty, so only lanes with a valid
  // column, n < gt[k], may use it in an address) and its valid columns gt[k]
  // (0 for the empty second block of a workgroup at the end of an odd number
  // of blocks)
  const int wb0 = kShared ? wave / WPB : 0;
  int hb[NBW], gt[NBW];
#pragma unroll
  for (int k = 0; k < NBW; ++k) {
    hb[k] = h0 + (wb0 + k) * bs;
    gt[k] = max(0, min(bs, gt_wg - (wb0 + k) * bs));
  }

  // B operand of the score MFMA: Q^T, head n of each block, loaded before the
  // page ids are staged so that the two memory round trips overlap.  16-bit:
  // features 32kk + 8grp .. + 8 (qb).  f32: lane group grp takes features
  // grp D/4 .. + D/4 as its share of every product, four per 16-byte chunk
  // (qf); any split of the contraction works as long as the A operand (K)
  // uses the same one.
  v8 qb[NBW][kF32 ? 1 : KK];
  f32x4 qf[NBW][kF32 ? QC : 1];
#pragma unroll
  for (int k = 0; k < NBW; ++k) {
    const bool live = n < gt[k];
    const char *qrow = static_cast<const char *>(p.q) +
                       ((int64_t)u.b * p.num_qo_heads + (live ? hb[k] + n : h0)) * D * E::kBytes;
    if constexpr (kF32) {
#pragma unroll
      for (int q4 = 0; q4 < QC; ++q4) {
        uint4 r = *reinterpret_cast<const uint4 *>(qrow + (grp * (D / 4) + 4 * q4) * 4);
        if (!live) r = make_uint4(0, 0, 0, 0);
        qf[k][q4] = __builtin_bit_cast(f32x4, r);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        uint4 r = *reinterpret_cast<const uint4 *>(qrow + (8 * grp) * 2 + kk * 64);
        if (!live) r = make_uint4(0, 0, 0, 0);
        qb[k][kk] = __builtin_bit_cast(v8, r);
      }
    }
  }

  __shared__ int32_t s_pages[kPageTable];
  const int slot0 = stage_unit_pages(p, s_pages, page_base, t_begin, t_end, NW * 64);

  // ALiBi slope of head n of each block (base-2 units): row t's score gains
  // slope2 * (t - (L - 1))
  float slope2[NBW];
#pragma unroll
  for (int k = 0; k < NBW; ++k)
    slope2[k] = (kMods && p.alibi && n < gt[k]) ? p.alibi[hb[k] + n] * kLog2e : 0.0f;

  f32x4 acc[NBW][MB];
  float m_run[NBW];  // running max (base 2) of head n; same in all 4 lane groups
  float l_run[NBW];  // this lane's share of the normaliser of head n
#pragma unroll
  for (int k = 0; k < NBW; ++k) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[k][mb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    m_run[k] = -INFINITY;
    l_run[k] = 0.0f;
  }

  char *wk = lds + wave * G::WAVE_LDS;   // this wave's K tile
  char *wv = wk + TT * G::ROWK;           // and V tile
  const float c = p.scale_log2;
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  // 16-bit V: this lane's address in each transposed read: row 4 grp + (n / 4)
  // of the 16-row half, features 4 (n % 4) .. + 3 of the 16-feature block.
  // f32 V: row 4 grp (+ i) and feature n (+ 16 mb), read directly.
  const int vt_off = kF32 ? (4 * grp) * G::ROWV + n * 4
                          : (4 * grp + (n >> 2)) * G::ROWV + (4 * (n & 3)) * 2;
  // where this lane's loaded 16 bytes go: row RPI * i + lane / LPR
  const int st_row = lane / G::LPR, st_col = (lane % G::LPR) * 16;

  // Custom mask of the tile at t0: its 32 bits start at bit B = row0 + t0 and
  // span bytes B/8 .. B/8 + 4.  mask_load issues one load instruction for
  // them with the tile's K/V loads (lanes 0-4, a byte each; bytes past the
  // mask's end read as 0); at compute time mask_word assembles the wave's
  // bytes into the tile's word (bit r for row t0 + r, the same in every
  // lane) and lane_bits picks the lane's rows (bit 4j + i for row
  // t0 + 16j + 4grp + i, j < JB).
  // Rows past the request (a prefetched tile, the tail of the last one) see
  // other bits and are cut by t_end.
  auto mask_load = [&](int t0) -> uint32_t {
    uint32_t v = 0;
    if constexpr (kMods) {
      if (p.mask) {
        const uint32_t byte = ((uint32_t)(u.row0 + t0) >> 3) + (uint32_t)lane;
        if (lane < 5 && byte < p.mask_bytes) v = p.mask[byte];
      }
    }
    return v;
  };
  auto mask_word = [&](int t0, uint32_t v) -> uint32_t {
    uint64_t w = 0;
#pragma unroll
    for (int k = 0; k < 5; ++k) w |= (uint64_t)__builtin_amdgcn_readlane(v, k) << (8 * k);
    return (uint32_t)(w >> ((uint32_t)(u.row0 + t0) & 7));  // bit r: row t0 + r
  };
  auto lane_bits = [&](uint32_t tile) -> uint32_t {
    const uint32_t lo = (tile >> (4 * grp)) & 0xFu;
    return JB == 2 ? lo | (((tile >> (16 + 4 * grp)) & 0xFu) << 4) : lo;
  };

  // K and V tiles as loaded -> this wave's LDS area
  auto store_tile = [&](const KVTile<G::NI> &T) {
#pragma unroll
    for (int i = 0; i < G::NI; ++i) {
      const int r = G::RPI * i + st_row;
      *reinterpret_cast<uint4 *>(wk + r * G::ROWK + st_col) = T.k[i];
      *reinterpret_cast<uint4 *>(wv + r * G::ROWV + st_col) = T.v[i];
    }
  };

  // One tile (rows t0 .. t0 + TT) for this wave's heads (each block's), from
  // the LDS area at ck (K rows, then V rows).
  // mbits: the lane's mask bits of the tile (lane_bits; unused without a mask).
  auto compute_tile = [&](const char *ck, int t0, uint32_t mbits) {
    const char *vt = ck + TT * G::ROWK + vt_off;
    // scores; A = K row 16j + n: features 32kk + 8grp .. + 8 (16-bit), or the
    // lane group's quarter of D, one feature per product (f32); each A
    // operand serves every block
    f32x4 s[NBW][JB];
#pragma unroll
    for (int j = 0; j < JB; ++j) {
#pragma unroll
      for (int k = 0; k < NBW; ++k) s[k][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      if constexpr (kF32) {
#pragma unroll
        for (int q4 = 0; q4 < QC; ++q4) {
          const f32x4 ka = *reinterpret_cast<const f32x4 *>(
              ck + (16 * j + n) * G::ROWK + (grp * (D / 4) + 4 * q4) * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int k = 0; k < NBW; ++k) s[k][j] = Mfma<F32>::mma4(ka[e], qf[k][q4][e], s[k][j]);
        }
      } else {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const uint4 ka = *reinterpret_cast<const uint4 *>(ck + (16 * j + n) * G::ROWK +
                                                            (32 * kk + 8 * grp) * 2);
#pragma unroll
          for (int k = 0; k < NBW; ++k)
            s[k][j] = M::mma(__builtin_bit_cast(v8, ka), qb[k][kk], s[k][j]);
        }
      }
    }
    // online softmax for head n of each block over the tile's rows
    // 16j + 4grp + i
    float pr[NBW][4 * JB];
#pragma unroll
    for (int k = 0; k < NBW; ++k) {
      float x[4 * JB];
      float tmax = -INFINITY;
#pragma unroll
      for (int j = 0; j < JB; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = t0 + 16 * j + 4 * grp + i;
          float v = s[k][j][i] * c;
          if constexpr (kMods) {
            if (p.alibi) v += slope2[k] * (float)(t - last_row);
            if (p.softcap2 > 0.0f) v = p.softcap2 * tanhf(v * p.softcap2_inv);
            if (t < t_lo) v = -INFINITY;
            if (p.mask && !((mbits >> (4 * j + i)) & 1u)) v = -INFINITY;
          }
          if (t >= t_end) v = -INFINITY;
          x[4 * j + i] = v;
          tmax = fmaxf(tmax, v);
        }
      tmax = rows4_max(tmax);
      const float m_new = fmaxf(m_run[k], tmax);
      const float ref = safe_ref(m_new);
      const float alpha = fast_exp2(m_run[k] - ref);
      float psum = 0.0f;
#pragma unroll
      for (int e = 0; e < 4 * JB; ++e) {
        pr[k][e] = fast_exp2(x[e] - ref);
        psum += pr[k][e];
      }
      l_run[k] = l_run[k] * alpha + psum;
      m_run[k] = m_new;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[k][mb] *= alpha;
    }
    if constexpr (kF32) {
      // O^T += V^T P^T over the 16 rows, 4 at a time: in product i, lane group
      // grp contributes row 4grp + i, so B is the lane's own probability pr[i]
      // and A is V[row 4grp + i][feature 16mb + n]
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a = *reinterpret_cast<const float *>(vt + i * G::ROWV + 64 * mb);
#pragma unroll
          for (int k = 0; k < NBW; ++k) acc[k][mb] = Mfma<F32>::mma4(a, pr[k][i], acc[k][mb]);
        }
    } else {
      v8 ph[NBW], pl[NBW];
#pragma unroll
      for (int k = 0; k < NBW; ++k) pack_probs<E>(pr[k], ph[k], pl[k]);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        // A = V^T: rows 16h + 4grp + r (r < 4) of feature 16mb + n, for h = 0, 1
        const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4 *)(vt + 32 * mb));
        const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4 *)(vt + 16 * G::ROWV + 32 * mb));
        typedef short s16x8 __attribute__((ext_vector_type(8)));
        const s16x8 a16 = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
        const v8 a = __builtin_bit_cast(v8, a16);
#pragma unroll
        for (int k = 0; k < NBW; ++k) {
          acc[k][mb] = M::mma(a, ph[k], acc[k][mb]);
          if constexpr (M::kSplitP) acc[k][mb] = M::mma(a, pl[k], acc[k][mb]);
        }
      }
    }
  };

  // Each wave stores its tile and computes it alone.
  auto compute = [&](const KVTile<G::NI> &T, int t0, uint32_t mraw) {
    store_tile(T);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    uint32_t mbits = 0;
    if constexpr (kMods)
      if (p.mask) mbits = lane_bits(mask_word(t0, mraw));
    compute_tile(wk, t0, mbits);
    // the reads above complete before the next tile overwrites the area
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  const int stride = NW * TT;
  int t0 = t_begin + wave * TT;
  if constexpr (kShared) {
    // Shared tiles: step s covers rows t_begin + s * stride ..; wave w loads
    // the step's tile w into its LDS area and computes tiles cw .. cw + NB - 1
    // for its block's heads.  Every wave runs every step (the barriers are the
    // workgroup's), loading clamped rows where its tile lies past the unit.
    // A custom mask's word of each tile is assembled by the wave that loaded
    // the tile and published in s_mask with it.  One register tile, reloaded
    // as soon as it is in LDS, so the next step's loads stream while this
    // step is computed.
    const int steps = t_begin < t_end ? (t_end - t_begin + stride - 1) / stride : 0;
    const int cw = (wave % WPB) * NB;
    if (steps > 0) {
      KVTile<G::NI> A;
      issue_tile<E, D, kNhd>(A, p, page_base, s_pages, slot0, kvh, t0, t_end, lane);
      uint32_t mA = mask_load(t0);
      for (int st = 0; st < steps; ++st) {
        store_tile(A);
        if constexpr (kMods)
          if (p.mask && lane == 0) s_mask[wave] = mask_word(t0 + st * stride, mA);
        if (st + 1 < steps) {
          issue_tile<E, D, kNhd>(A, p, page_base, s_pages, slot0, kvh, t0 + (st + 1) * stride,
                                 t_end, lane);
          mA = mask_load(t0 + (st + 1) * stride);
        }
        __syncthreads();
        const int ts = t_begin + st * stride;
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          const int tc = ts + (cw + i) * TT;
          uint32_t mbits = 0;
          if constexpr (kMods)
            if (p.mask) mbits = lane_bits(s_mask[cw + i]);
          if (tc < t_end && gt[0] > 0) compute_tile(lds + (cw + i) * G::WAVE_LDS, tc, mbits);
        }
        __syncthreads();  // the step's tiles are read by every wave before they are replaced
      }
    }
  } else {
    // The wave's tiles: tile k starts at row t0 + k * stride, k < n_tiles.
    // Under a custom mask only the tiles holding a kept row are loaded and
    // computed (live_tile); a skipped tile would leave the state as it is.
    const int n_tiles = t0 < t_end ? (t_end - t0 + stride - 1) / stride : 0;
    uint64_t live = ~0ull;  // bit i: tile win0 + i may hold a kept row
    int win0 = 0;
    // the live bits of tiles k0 .. k0 + 63 (a superset: each lane ORs the
    // five mask bytes that cover its tile's 32 bits; bytes past the mask's
    // end read as 0)
    auto scan_mask = [&](int k0) -> uint64_t {
      uint32_t any = 0;
      if constexpr (kMods) {
        const int t = t0 + (k0 + lane) * stride;
        if (k0 + lane < n_tiles) {
          const uint32_t b0 = (uint32_t)(u.row0 + t) >> 3;
#pragma unroll
          for (int e = 0; e < 5; ++e)
            if (b0 + e < p.mask_bytes) any |= p.mask[b0 + e];
        }
      }
      return __ballot(any != 0);
    };
    if constexpr (kMods)
      if (p.mask) live = scan_mask(0);
    // the first live tile at or after k (k <= n_tiles; n_tiles if none)
    auto live_tile = [&](int k) -> int {
      if constexpr (kMods) {
        if (p.mask) {
          while (k < n_tiles) {
            if (k >= win0 + 64) {
              win0 = k;
              live = scan_mask(k);
            }
            const uint64_t m = live >> (k - win0);
            if (m) return min(k + (int)__builtin_ctzll(m), n_tiles);
            k = win0 + 64;
          }
          return n_tiles;
        }
      }
      return k;
    };
    auto row_of = [&](int k) { return t0 + k * stride; };
    int ka = live_tile(0);
    if (ka < n_tiles) {
      KVTile<G::NI> A;
      issue_tile<E, D, kNhd>(A, p, page_base, s_pages, slot0, kvh, row_of(ka), t_end, lane);
      uint32_t mA = mask_load(row_of(ka));
      if constexpr (kPipe && !kMods) {
        // every tile, two in flight, at a fixed stride (the live-tile form
        // below measured ~1% slower here); the next tile's loads go out
        // unconditionally: past the wave's last tile they read the unit's
        // last row again (clamped, in bounds, from cache), which keeps every
        // wait for a tile's data exact
        KVTile<G::NI> B;
        int ta = t0;
        while (true) {
          issue_tile<E, D, kNhd>(B, p, page_base, s_pages, slot0, kvh, ta + stride, t_end, lane);
          compute(A, ta, 0);
          ta += stride;
          if (ta >= t_end) break;
          issue_tile<E, D, kNhd>(A, p, page_base, s_pages, slot0, kvh, ta + stride, t_end, lane);
          compute(B, ta, 0);
          ta += stride;
          if (ta >= t_end) break;
        }
      } else if constexpr (kPipe) {
        // the live tiles, two in flight, loaded the same way
        KVTile<G::NI> B;
        uint32_t mB = 0;
        while (true) {
          const int kb = live_tile(ka + 1);
          issue_tile<E, D, kNhd>(B, p, page_base, s_pages, slot0, kvh, row_of(kb), t_end, lane);
          mB = mask_load(row_of(kb));
          compute(A, row_of(ka), mA);
          if (kb >= n_tiles) break;
          ka = live_tile(kb + 1);
          issue_tile<E, D, kNhd>(A, p, page_base, s_pages, slot0, kvh, row_of(ka), t_end, lane);
          mA = mask_load(row_of(ka));
          compute(B, row_of(kb), mB);
          if (ka >= n_tiles) break;
        }
      } else {
        // One register tile (D = 256, or two head blocks): once it is in LDS
        // its registers are free, so the next tile's loads are issued before
        // the current one is computed and stream meanwhile.
        while (true) {
          store_tile(A);
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
          uint32_t mbits = 0;
          if constexpr (kMods)
            if (p.mask) mbits = lane_bits(mask_word(row_of(ka), mA));
          const int kn = live_tile(ka + 1);
          if (kn < n_tiles) {
            issue_tile<E, D, kNhd>(A, p, page_base, s_pages, slot0, kvh, row_of(kn), t_end, lane);
            mA = mask_load(row_of(kn));
          }
          compute_tile(wk, row_of(ka), mbits);
          // the reads above complete before the next tile overwrites the area
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
          ka = kn;
          if (ka >= n_tiles) break;
        }
      }
    }
  }

  // ---- merge the four lane groups' normalisers, then the waves
#pragma unroll
  for (int k = 0; k < NBW; ++k) l_run[k] = rows4_sum(l_run[k]);
  __syncthreads();  // every wave is done with its V area; reuse it for the merge
  float *s_acc = reinterpret_cast<float *>(lds);  // [NW][NBW * 16][ACC_ROW]
#pragma unroll
  for (int k = 0; k < NBW; ++k) {
    if (n < gt[k]) {
      const int row = wave * NBW * 16 + k * 16 + n;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          s_acc[row * G::ACC_ROW + 16 * mb + 4 * grp + i] = acc[k][mb][i];
      if (grp == 0) {
        s_m[wave][k * 16 + n] = m_run[k];
        s_l[wave][k * 16 + n] = l_run[k];
      }
    }
  }
  __syncthreads();
  // workgroup head hh = head g of block kb = hh / bs: merged over the WPB
  // waves that hold it (waves kb * WPB .. with shared tiles, where each wave
  // holds one block; else every wave, as its block kb); each thread takes
  // four adjacent features, read from LDS and stored at once
  constexpr int D4 = D / 4;
  for (int idx = tid; idx < gt_wg * D4; idx += NW * 64) {
    const int hh = idx / D4;
    const int d = (idx - hh * D4) * 4;
    const int kb = NB == 1 ? 0 : hh / bs;
    const int w0 = kShared ? kb * WPB : 0;
    const int col = (kShared ? 0 : kb) * 16 + (hh - kb * bs);
    float Mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < WPB; ++w) Mx = fmaxf(Mx, s_m[w0 + w][col]);
    const float ref = safe_ref(Mx);
    float lsum = 0.0f;
    float a[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int w = 0; w < WPB; ++w) {
      const float sw = fast_exp2(s_m[w0 + w][col] - ref);
      lsum += s_l[w0 + w][col] * sw;
      const float4 v = *reinterpret_cast<const float4 *>(
          &s_acc[((w0 + w) * NBW * 16 + col) * G::ACC_ROW + d]);
      a[0] += v.x * sw;
      a[1] += v.y * sw;
      a[2] += v.z * sw;
      a[3] += v.w * sw;
    }
    emit<E>(p, u, h0 + hh, d, Mx, lsum, a);
  }
  // merge depth 16 where the main loop's register peak already covers it
  // (D >= 128); 8 at D = 64, where 16 would cost occupancy
  finish_split<E, (D >= 128 ? 16 : 8)>(p, u, plane, h0, gt_wg, NW, s_stat, &s_last,
                                        reinterpret_cast<float *>(lds), G::LDS / 4);
}

// ------------------------------------------------------------ gather hook
//
// Test-only: the page-table gather exactly as the decode kernel performs it,
// so a test can compare the rows the kernel loads with an independent gather
// bit for bit.  Same work decomposition (one workgroup per split unit and KV
// head, units from find_unit), same LDS page staging (stage_unit_pages), same
// per-wave tile walk (tile t0 = t_begin + wave * TT, then every NW * TT rows)
// and the same loads (issue_tile, rows past the unit clamped to its last
// row).  Instead of computing, each wave writes the rows it loaded that lie
// inside the unit to out[(row0_b + t) * Hkv + kvh, :], row0_b = L_0 + .. +
// L_{b-1}.  p.k and p.v both point at the store being gathered.
template <class E, int D, bool kNhd>
__global__ __launch_bounds__(mfma_waves(D) * 64) void gather_tiles_kernel(const DecodeParams p,
                                                                          char *out,
                                                                          int64_t out_rows) {
  using G = MfmaGeom<E, D>;
  constexpr int NW = G::NW, TT = G::TT;
  const int unit = blockIdx.x / p.planes;
  const int kvh = blockIdx.x - unit * p.planes;  // one query head per KV head: planes = Hkv
  UnitInfo u;
  if (!find_unit<true>(p, unit, u)) return;
  const int t_begin = __builtin_amdgcn_readfirstlane(u.lo + u.c * p.chunk);
  const int t_end = __builtin_amdgcn_readfirstlane(min(u.L, t_begin + p.chunk));
  const int32_t page_base = __builtin_amdgcn_readfirstlane(u.page_base);
  __shared__ int32_t s_pages[kPageTable];
  const int slot0 = stage_unit_pages(p, s_pages, page_base, t_begin, t_end, NW * 64);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int r0 = lane / G::LPR, col = (lane % G::LPR) * 16;
  for (int t0 = t_begin + wave * TT; t0 < t_end; t0 += NW * TT) {
    KVTile<G::NI> T;
    issue_tile<E, D, kNhd>(T, p, page_base, s_pages, slot0, kvh, t0, t_end, lane);
#pragma unroll
    for (int i = 0; i < G::NI; ++i) {
      const int t = t0 + G::RPI * i + r0;
      const int64_t orow = (int64_t)u.row0 + t;
      if (t < t_end && orow < out_rows)
        *reinterpret_cast<uint4 *>(out + ((orow * p.num_kv_heads + kvh) * D) * E::kBytes +
                                   col) = T.k[i];
    }
  }
}

}  // namespace fa
