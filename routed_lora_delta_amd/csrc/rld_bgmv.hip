// Routed BGMV ("Function apply_lora_bgmv"; lora_delta.rs, apply_lora_bgmv):
// every row i of a batch names an adapter slot s = seq_slot[i]; the shrink writes
// xa[i] = bf16(x_i @ A_s^T) and the expand folds bf16(xa[i] @ B_s^T), scaled in
// fp32 after the rounding, into the row's output.
//
// Work is slot-grouped: an item serves one slot and all rows that name it, so
// each slot's A_s / B_s tile is streamed from HBM once per call instead of once
// per row.  The row list of a slot is rebuilt by every item from seq_slot (no
// host read), in ascending row order.
//
//   shrink item  (slot, k_in chunk, up to 64 columns of xa).  Each of the NW
//                waves (4 or 8, by (k_in, max_rank)) owns every NW-th 32-wide K
//                step of the chunk and issues all of its A fragments at once,
//                then the x fragments of up to 64 (8 waves: 128) rows at once.
//                The waves' partial sums are added in wave order.  With one chunk the sum is rounded to xa right away;
//                otherwise it is stored as an fp32 partial [chunk][row][col]
//                in the workspace (zeros for base rows), and a second, small
//                kernel adds each row's chunks in chunk order and writes xa.
//                The chunk length depends only on (k_in, max_rank), so
//                a row's summation order is the same whatever the batch holds:
//                a batched call is bit-identical to one-row calls.
//   expand item  (slot, 256 output columns).  B_s rows of the tile are
//                the MFMA A operands; rows of the slot stream through as the B
//                operand (16 rows per MFMA).  The B tile, the base values and
//                the xa rows of a 64-row pass go out in one round of loads,
//                deltas are rounded to BF16 into LDS, and the fold writes
//                16-byte coalesced vectors.  Grids too large for one round of the
//                classic item's registers take a lean item that holds the B
//                tile and moves rows in passes of 16 (same bits).
//
// rld_bgmv launches the shrink (and its reduce), then the expand, on the
// caller's stream.
#include <mutex>
#include <type_traits>

#include "rld_device.hpp"
#include "rld_internal.hpp"

namespace rld {

constexpr int kReduceThreads = 64;  // chunk reduce: one-wave blocks, one element a thread
constexpr int kChunkSteps = 16;  // 32-wide K steps of the longest chunk (512)
constexpr int kListCap = 512;    // rows collected per pass over seq_slot
constexpr int kExpRows = 64;     // rows per fold pass of the expand

// Shape of a shrink block of NW waves: KS K steps per wave, batches of QT
// 16-row subtiles (the x fragments of a batch are QT * KS = 16 per lane either
// way), and MR subtiles per round of the wave reduce in LDS.
template <int NT, int NW, int QTO = 0>
struct ShrinkShape {
  static_assert(NW == 4 || NW == 8, "four or eight waves");
  static constexpr int kThreads = NW * kWave;
  static constexpr int KS = kChunkSteps / NW;
  static constexpr int QT = QTO ? QTO : 16 / KS;
  // 64-row batches (QTO = 4) keep the LDS of two subtiles' wave sums, so that
  // three blocks share a CU
  static constexpr int MR = QTO ? 2 : (NW * NT * 4 <= 64 ? 4 : 2);
  static_assert(KS * NW * 32 >= 512, "a chunk is at most 512 elements");
};

// Kernel arguments; device addresses are kept as integers and read through
// the global-pointer accessors.
struct BgmvArgs {
  uint64_t x_, seq_, atab_, btab_, stab_;
  uint64_t partial_;  // [nch][n][R] fp32 (k split only): the workspace
  uint64_t xa_, out_;
  // Unrouted mode (dense != 0): one pair for every row; items take contiguous
  // row tiles instead of a slot's rows, and seq_slot and the tables are unused.
  uint64_t a_dense, b_dense;
  float scale_dense;
  uint32_t dense;
  uint32_t xs, n, max_loras, k_in, n_out, R, kc, nch;
  uint32_t ncg;  // shrink column groups of 16*NT xa columns
  uint32_t os;
  __device__ const RLD_GLOBAL uint16_t* x() const { return gp<const uint16_t>(x_); }
  __device__ const RLD_GLOBAL int32_t* seq_slot() const { return gp<const int32_t>(seq_); }
  __device__ const RLD_GLOBAL uint64_t* a_table() const { return gp<const uint64_t>(atab_); }
  __device__ const RLD_GLOBAL uint64_t* b_table() const { return gp<const uint64_t>(btab_); }
  __device__ const RLD_GLOBAL float* scale_table() const { return gp<const float>(stab_); }
  __device__ RLD_GLOBAL float* partial() const { return gp<float>(partial_); }
  __device__ RLD_GLOBAL uint16_t* xa() const { return gp<uint16_t>(xa_); }
  __device__ RLD_GLOBAL uint16_t* out() const { return gp<uint16_t>(out_); }
};

template <int NT, int NW, int QTO = 0>
struct ShrinkSmem {
  int rows[kListCap];
  int wcount[NW];
  floatx4 red[NW][ShrinkShape<NT, NW, QTO>::MR * NT][kWave];
};

// Expand item of 64*MT output columns (16*MT per wave).
template <int MT>
struct ExpandSmem {
  static constexpr int kCols = 64 * MT;
  static constexpr int kStride = kCols + 8;  // LDS row stride of the delta tile
  int rows[kListCap];
  int wcount[4];
  __attribute__((aligned(16))) uint16_t dl[kExpRows * kStride];
};

// Lean expand item (256 output columns, rows in passes of 16): a fraction of
// the registers and LDS of ExpandSmem<4>'s item, so that six blocks share a CU
// and a decode call's (column tile, slot) grid goes out in one round.
constexpr int kLeanRows = 16;   // rows per pass of the lean expand item (16 or 32)
struct ExpandLeanSmem {
  static constexpr int kCols = 256;
  static constexpr int kStride = kCols + 8;
  static constexpr int kRows = kLeanRows;
  int rows[kListCap];
  int wcount[4];
  __attribute__((aligned(16))) uint16_t dl[kRows * kStride];
};

// One-pass fold (rld_bgmv / rld_bgmv_multi at max_rank <= 16, k_in <= 4096,
// decode-sized batches): one launch, no workspace.  A block takes (slot s,
// 512 output columns) and first recomputes the xa of s's rows itself, in the
// summation order of the k-split shrink and its chunk reduce: its sixteen
// waves take one 256-wide chunk each and run, inside the wave, the four
// chains of the shrink's four waves (steps w, w+4, w+8, w+12 of the chunk)
// and their wave-order sum; the chunk sums meet in LDS and are added in chunk
// order, then rounded.  Every block of a slot therefore holds the xa bits the
// three launches would have written, and expands its columns from LDS with
// the expand's arithmetic.  The slot's A tile is read by each of its column
// groups (from cache after the first; the groups of a slot share an XCD).
constexpr int kOpThreads = 1024;
constexpr int kOpWaves = kOpThreads / kWave;
constexpr int kOpCols = 512;       // output columns per item (32 per wave)
constexpr int kOpChunk = 256;      // the k-split chunk at max_rank <= 16
constexpr int kOpMaxRows = 256;    // n of the calls that take this path
struct OnePassSmem {
  static constexpr int kStride = kOpCols + 8;
  static constexpr int kStageRow = 33;  // uint4 per staged A row (32 + 1: no bank conflicts)
  int rows[kOpMaxRows];
  int wcount[kOpWaves];
  __attribute__((aligned(16))) uint16_t xs[16 * 16];  // the batch's xa, row-major
  union {
    // each wave's chunk of the A tile (16 rows x 512 bytes), staged once
    uint4 stage[kOpWaves][16 * kStageRow];
    struct {
      floatx4 red[kOpWaves][kWave];  // chunk sums of a 16-row batch
      __attribute__((aligned(16))) uint16_t dl[16 * kStride];
    } w;
  } u;
};

__device__ __forceinline__ bool slot_active(const BgmvArgs& a, int s) {
  if (s < 0 || (uint32_t)s >= a.max_loras) return false;
  const uint64_t ta = a.a_table()[s], tb = a.b_table()[s];  // both in flight together
  return ta != 0ull && tb != 0ull;
}

// Appends to `rows` (LDS) the rows of slot s from seq_slot[*pos ...], until
// n is reached or the list cannot take another NW*64; advances *pos.  Returns
// the count (the same in every thread).  key0 is this thread's seq_slot entry
// of the first NW*64 rows (row threadIdx.x), loaded by the caller ahead of its
// tile loads so the first scan does not wait behind them.
template <int NW = 4>
__device__ __forceinline__ int collect_slot_rows(const RLD_GLOBAL int32_t* seq_slot, uint32_t n,
                                                 uint32_t* pos, int s, int* rows, int* wcount,
                                                 int key0) {
  constexpr int NTH = NW * kWave;
  int cnt = 0;
  while (*pos < n && cnt <= kListCap - NTH) {
    const uint32_t row = *pos + threadIdx.x;
    const int key = *pos == 0 ? key0 : (row < n ? seq_slot[row] : -1);
    cnt += append_hits<NW>(row < n && key == s, row, rows, cnt, wcount);
    *pos += NTH;
  }
  return cnt;
}

// This thread's seq_slot entry among the first blockDim rows (-1 past n).  The
// load is unconditional (a row < n is always readable) so that it stays in the
// prologue, ahead of the tile loads.
__device__ __forceinline__ int first_key(const RLD_GLOBAL int32_t* seq_slot, uint32_t n) {
  const int k = seq_slot[min(threadIdx.x, n - 1)];
  issue_point();  // issued before any load that follows
  return threadIdx.x < n ? k : -1;
}

// Table entries of a slot s < max_loras, read together (one round trip).
struct SlotEntry {
  uint64_t a, b;
  float scale;
  __device__ bool active() const { return a != 0ull && b != 0ull; }
};

__device__ __forceinline__ SlotEntry slot_entry(const BgmvArgs& a, int s) {
  SlotEntry e;
  e.a = a.a_table()[s];
  e.b = a.b_table()[s];
  e.scale = a.scale_table()[s];
  return e;
}

// Rows of the shrink / expand tiles of the unrouted mode: a shrink tile is
// one batch of its block (64 rows with four waves, 128 with eight).
__host__ __device__ constexpr int dense_shrink_rows(int nw) { return nw == 8 ? 128 : 64; }
constexpr int kDenseExpandRows = 128;

// Unrouted mode: rows [r0, r0 + cnt) of a tile into the LDS row list.
__device__ __forceinline__ int dense_tile_rows(uint32_t r0, uint32_t n, int tile, int* rows) {
  const int cnt = (int)min((uint32_t)tile, n - r0);
  for (int i = threadIdx.x; i < cnt; i += blockDim.x) rows[i] = (int)(r0 + i);
  __syncthreads();
  return cnt;
}

// Shrink item w (slot-major over (slot, chunk, column group)); the group
// covers xa columns [16*NT*cg, 16*NT*(cg+1)).
template <int NT, int NW, int QTO = 0>
__device__ void shrink_item(const BgmvArgs& a, uint32_t w, ShrinkSmem<NT, NW, QTO>& sm) {
  using SS = ShrinkShape<NT, NW, QTO>;
  constexpr int NTH = SS::kThreads, KS = SS::KS, QT = SS::QT, MR = SS::MR;
  const uint32_t n = a.n, R = a.R, nchunks = a.nch, ncg = a.ncg;
  const uint32_t cg = w % ncg;
  const uint32_t c = (w / ncg) % nchunks;
  const int s = (int)(w / (ncg * nchunks));  // slot, or row tile in the unrouted mode
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const uint32_t col0 = cg * 16u * NT;

  // The block's seq_slot entries and the slot's table entries go out first.
  int key0 = -1;
  SlotEntry ent;
  if (a.dense) {
    ent.a = a.a_dense;
    ent.b = a.b_dense;
    ent.scale = a.scale_dense;
  } else {
    key0 = first_key(a.seq_slot(), n);
    ent = slot_entry(a, s);
  }

  // Zeros for base rows, by the items of the last slot (usually cold, so these
  // blocks have nothing else to do): the item of chunk c and column group cg
  // writes the base rows' xa columns of the group (no k split) or their
  // partials of chunk c (so the chunk reduce needs no routing).  One row per
  // thread; the first NTH rows' slots are key0.
  if (!a.dense && (uint32_t)s == a.max_loras - 1) {
    const uint32_t c1 = min(col0 + 16u * NT, R);
    for (uint32_t r0 = 0; r0 < n; r0 += NTH) {
      const uint32_t row = r0 + threadIdx.x;
      const int key = r0 == 0 ? key0 : (row < n ? a.seq_slot()[row] : 0);
      if (row >= n || slot_active(a, key)) continue;
      if (nchunks == 1) {
        for (uint32_t cc = col0; cc < c1; cc += 8) store16(a.xa() + (size_t)row * R + cc, zero16());
      } else {
        RLD_GLOBAL float* pp = a.partial() + ((size_t)c * n + row) * R;
        for (uint32_t cc = col0; cc < c1; cc += 4)
          store16(reinterpret_cast<RLD_GLOBAL uint16_t*>(pp + cc), zero16());
      }
    }
  }
  if (!ent.active()) return;

  const RLD_GLOBAL uint16_t* A = gp<const uint16_t>(ent.a);
  const int lg = lane >> 4;
  const int cl = lane & 15;
  const uint32_t kb = c * a.kc;
  const uint32_t ke = min(kb + a.kc, a.k_in);
  const uint32_t nsteps = (ke - kb + 31) / 32;

  // K steps of this wave: wave, wave + NW, ... of the chunk
  uint32_t kof[KS];
  bool kok[KS];
#pragma unroll
  for (int i = 0; i < KS; ++i) {
    const uint32_t st = wave + NW * i;
    kof[i] = kb + st * 32 + lg * 8;
    kok[i] = st < nsteps && kof[i] < ke;
  }

  // Rows b0 .. b0 + 16*QT - 1 of the slot's list: the A fragments of this
  // wave's K steps for the NT column tiles, then the x fragments of all QT
  // subtiles, in one round of loads (unconditional A loads: out-of-range
  // lanes read the chunk's first element of row 0).  The slot's table entry
  // arrived with its seq_slot entries, so nothing is gained by issuing A
  // before the row scan.  Subtiles go through the wave reduce MR at a time;
  // (subtile, column tile) p of a round is added by wave p % NW.
  auto batch = [&](int b0, int cnt) {
    const int nb = min(cnt - b0, QT * 16);
    const int nmt = (nb + 15) >> 4;
    uint4 bop[NT][KS];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const uint32_t col = col0 + 16u * j + cl;
      const RLD_GLOBAL uint16_t* Arow = A + (size_t)(col < R ? col : 0) * a.k_in;
#pragma unroll
      for (int i = 0; i < KS; ++i)
        bop[j][i] = load16((col < R && kok[i]) ? Arow + kof[i] : A + kb);
    }
    uint4 xf[QT][KS];
#pragma unroll
    for (int q = 0; q < QT; ++q) {
      const int li = q * 16 + cl;
      const bool ok = li < nb;
      const RLD_GLOBAL uint16_t* xr = a.x() + (size_t)(ok ? sm.rows[b0 + li] : 0) * a.xs;
#pragma unroll
      for (int i = 0; i < KS; ++i)
        xf[q][i] = (q < nmt && ok && kok[i]) ? load16(xr + kof[i]) : zero16();
    }
    issue_point();
    // k past the chunk contributes nothing; columns past max_rank are
    // computed from clamped reads and never stored
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int i = 0; i < KS; ++i)
        if (!kok[i]) bop[j][i] = zero16();
#pragma unroll
    for (int h = 0; h < QT / MR; ++h) {
      if (h * MR >= nmt) break;
#pragma unroll
      for (int qq = 0; qq < MR; ++qq) {
        const int q = h * MR + qq;
        if (q < nmt) {
#pragma unroll
          for (int j = 0; j < NT; ++j) {
            floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < KS; ++i) acc = mfma_bf16_16x16x32(xf[q][i], bop[j][i], acc);
            sm.red[wave][qq * NT + j][lane] = acc;
          }
        }
      }
      __syncthreads();
      // (the lane index through an empty asm: the store addresses below are
      // computed here, not hoisted out of the batch and held)
      int tl = lane;
      asm volatile("" : "+v"(tl));
#pragma unroll
      for (int p = wave; p < MR * NT; p += NW) {
        const int qq = p / NT, j = p % NT;
        const int q = h * MR + qq;
        if (q < nmt) {
          const uint32_t col = col0 + 16u * j + (uint32_t)(tl & 15);
          floatx4 sum = sm.red[0][p][lane];
#pragma unroll
          for (int v = 1; v < NW; ++v) sum += sm.red[v][p][lane];
          if (col < R) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int li = q * 16 + 4 * (tl >> 4) + i;
              if (li < nb) {
                const uint32_t row = (uint32_t)sm.rows[b0 + li];
                if (nchunks == 1)
                  a.xa()[(size_t)row * R + col] = (uint16_t)f32_to_bf16(sum[i]);
                else
                  a.partial()[((size_t)c * n + row) * R + col] = sum[i];
              }
            }
          }
        }
      }
      __syncthreads();
    }
  };

  if constexpr (QTO == 0) {
    if (a.dense) {
      constexpr int kTile = dense_shrink_rows(NW);
      static_assert(kTile == QT * 16, "an unrouted tile is one batch");
      const int cnt = dense_tile_rows((uint32_t)s * kTile, n, kTile, sm.rows);
      batch(0, cnt);
      return;
    }
  }
  // The usual case, straight-line: at most NTH rows (their seq_slot entries
  // are key0, so the scan issues no load that would wait behind the A tile)
  // and at most one batch of them on this slot.
  if (n <= (uint32_t)NTH) {
    const int cnt = append_hits<NW>(key0 == s, threadIdx.x, sm.rows, 0, sm.wcount);
    if (cnt <= QT * 16) {
      if (cnt > 0) batch(0, cnt);
      return;
    }
  }
  uint32_t pos = 0;
  int cnt = collect_slot_rows<NW>(a.seq_slot(), n, &pos, s, sm.rows, sm.wcount, key0);
  for (;;) {
    for (int b0 = 0; b0 < cnt; b0 += QT * 16) batch(b0, cnt);
    if (pos >= n) break;
    cnt = collect_slot_rows<NW>(a.seq_slot(), n, &pos, s, sm.rows, sm.wcount, key0);
  }
}

// Expand item (slot s, 64*MT output columns from j0).  NKS = ceil(max_rank/32).
// With zcount = 2 or 4 (routed launches over more than 64 rows) the slot's rows
// of a decode batch are split between that many items: part z folds rows
// [z * P, (z + 1) * P) of the slot's list, P = 128 / zcount, so that a heavily
// routed slot's rows run beside each other instead of one batch after another
// (each row's arithmetic is the same either way).
template <int NKS, int MT>
__device__ void expand_item(const BgmvArgs& a, int s, uint32_t j0, ExpandSmem<MT>& sm,
                            uint32_t zpart = 0, uint32_t zcount = 1) {
  constexpr int kCols = ExpandSmem<MT>::kCols;
  constexpr int kStride = ExpandSmem<MT>::kStride;
  constexpr int kRowVecs = kCols / 8;            // 16-byte vectors per row of the tile
  constexpr int kRowsPerPass = 256 / kRowVecs;   // rows the block folds per pass
  constexpr int kFoldVecs = kExpRows / kRowsPerPass;
  const uint32_t n = a.n, R = a.R, n_out = a.n_out, os = a.os;
  // seq_slot entries and the slot's table entries first (one round trip)
  int key0 = -1;
  SlotEntry ent;
  if (a.dense) {
    ent.a = a.a_dense;
    ent.b = a.b_dense;
    ent.scale = a.scale_dense;
  } else {
    key0 = first_key(a.seq_slot(), n);
    ent = slot_entry(a, s);
  }
  if (!ent.active()) return;
  const RLD_GLOBAL uint16_t* B = gp<const uint16_t>(ent.b);
  const float scale = ent.scale;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lg = lane >> 4;
  const int cl = lane & 15;
  // fold mapping: vector i of a thread is row frow + kRowsPerPass*i, columns c8 .. c8+7
  const int frow = threadIdx.x / kRowVecs;
  const int c8 = (threadIdx.x % kRowVecs) * 8;
  const bool fcol_ok = j0 + c8 < n_out;

  // rows b0 .. min(b0 + 64, cnt) - 1 of the slot's list
  auto batch = [&](int b0, int cnt) {
    const int nb = min(cnt - b0, kExpRows);
    // One round of loads: the B_s rows of this wave's 16*MT columns as MFMA A
    // operands (unconditional: out-of-range lanes read B's first element),
    // the batch's base values and its xa rows.  The slot's table entry came
    // with its seq_slot entries, so B gains nothing by going out before the
    // row scan.
    uint4 aop[MT][NKS];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const uint32_t col = j0 + wave * 16 * MT + m * 16 + cl;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const uint32_t k = ks * 32 + lg * 8;
        aop[m][ks] = load16((col < n_out && k < R) ? B + (size_t)col * R + k : B);
      }
    }
    uint4 bv[kFoldVecs];
#pragma unroll
    for (int i = 0; i < kFoldVecs; ++i) {
      const int rl = frow + kRowsPerPass * i;
      bv[i] = (rl < nb && fcol_ok) ? load16(a.out() + (size_t)sm.rows[b0 + rl] * os + j0 + c8)
                                   : zero16();
    }
    uint4 bop[4][NKS];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int li = p * 16 + cl;
      const bool ok = li < nb;
      const RLD_GLOBAL uint16_t* xr = a.xa() + (size_t)(ok ? sm.rows[b0 + li] : 0) * R;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const uint32_t k = ks * 32 + lg * 8;
        bop[p][ks] = (p * 16 < nb && ok && k < R) ? load16(xr + k) : zero16();
      }
    }
    issue_point();
    // k past max_rank contributes nothing (xa operand already zero there);
    // columns past n_out are computed from clamped reads and never stored
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        if (ks * 32 + lg * 8 >= (int)R) aop[m][ks] = zero16();
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      if (p * 16 < nb) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) acc = mfma_bf16_16x16x32(aop[m][ks], bop[p][ks], acc);
          // lane holds delta[row p*16+cl][cols m*16 + 4*lg .. +3] of this wave's slice
          const uint32_t d01 = pack_bf16x2(acc[0], acc[1]);
          const uint32_t d23 = pack_bf16x2(acc[2], acc[3]);
          *reinterpret_cast<uint2*>(
              &sm.dl[(p * 16 + cl) * kStride + wave * 16 * MT + m * 16 + 4 * lg]) =
              make_uint2(d01, d23);
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kFoldVecs; ++i) {
      const int rl = frow + kRowsPerPass * i;
      if (rl < nb && fcol_ok) {
        const uint4 dv = *reinterpret_cast<const uint4*>(&sm.dl[rl * kStride + c8]);
        store16(a.out() + (size_t)sm.rows[b0 + rl] * os + j0 + c8, fold8(bv[i], dv, scale));
      }
    }
    __syncthreads();
  };

  if (a.dense) {  // s is the row tile
    const int cnt = dense_tile_rows((uint32_t)s * kDenseExpandRows, n, kDenseExpandRows, sm.rows);
    batch(0, cnt);
    if (cnt > kExpRows) batch(kExpRows, cnt);
    return;
  }
  // The usual case, straight-line: at most 256 rows (their seq_slot entries
  // are key0) and at most 128 of them on this slot.
  if (n <= 256) {
    const int cnt = append_hits(key0 == s, threadIdx.x, sm.rows, 0, sm.wcount);
    if (cnt <= 2 * kExpRows) {
      if (zcount == 1) {
        if (cnt > 0) batch(0, cnt);
        if (cnt > kExpRows) batch(kExpRows, cnt);
      } else {
        const int part = 2 * kExpRows / (int)zcount;
        const int r0 = (int)zpart * part;
        if (r0 < cnt) batch(r0, min(r0 + part, cnt));
      }
      return;
    }
  }
  if (zpart != 0) return;  // part 0 folds every batch of the general case
  uint32_t pos = 0;
  while (pos < n) {
    const int cnt = collect_slot_rows(a.seq_slot(), n, &pos, s, sm.rows, sm.wcount, key0);
    for (int b0 = 0; b0 < cnt; b0 += kExpRows) batch(b0, cnt);
  }
}

// Lean expand item (slot s, 256 output columns from j0; routed mode only).
// The same per-row arithmetic as expand_item (one MFMA chain over max_rank
// per 16 x 16 tile, BF16 rounding, the fold), so results are bit-identical;
// rows go through in passes of 16, the next pass's xa and base values in
// flight while the current pass folds.
template <int NKS>
__device__ void expand_lean_item(const BgmvArgs& a, int s, uint32_t j0, ExpandLeanSmem& sm) {
  constexpr int kStride = ExpandLeanSmem::kStride;
  constexpr int kRows = ExpandLeanSmem::kRows;
  const uint32_t n = a.n, R = a.R, n_out = a.n_out, os = a.os;
  const int key0 = first_key(a.seq_slot(), n);
  const SlotEntry ent = slot_entry(a, s);
  if (!ent.active()) return;
  const RLD_GLOBAL uint16_t* B = gp<const uint16_t>(ent.b);
  const float scale = ent.scale;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lg = lane >> 4;
  const int cl = lane & 15;
  // fold mapping: 32 vectors of 8 columns per row; vector i of a thread is
  // row frow + 8*i of the pass
  const int frow = threadIdx.x >> 5;
  const int c8 = (threadIdx.x & 31) * 8;
  const bool fcol_ok = j0 + c8 < n_out;

  int cnt;
  uint32_t pos = 0;
  if (n <= 256) {
    cnt = append_hits(key0 == s, threadIdx.x, sm.rows, 0, sm.wcount);
    pos = n;
  } else {
    cnt = collect_slot_rows(a.seq_slot(), n, &pos, s, sm.rows, sm.wcount, key0);
  }
  if (cnt == 0 && pos >= n) return;

  // The B rows of this wave's 64 columns as MFMA A operands, once per item
  // (unconditional: out-of-range lanes read B's first element).
  uint4 aop[4][NKS];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const uint32_t col = j0 + wave * 64 + m * 16 + cl;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const uint32_t k = ks * 32 + lg * 8;
      aop[m][ks] = load16((col < n_out && k < R) ? B + (size_t)col * R + k : B);
    }
  }
  // xa fragments and base values of rows b0 .. b0+15 of the list
  constexpr int PT = kRows / 16;  // 16-row subtiles of a pass
  constexpr int FV = kRows / 8;   // fold vectors of a thread per pass
  auto load_xa = [&](int b0, int cnt_, uint4 (&bop)[PT][NKS]) {
#pragma unroll
    for (int p = 0; p < PT; ++p) {
      const bool ok = p * 16 + cl < cnt_ - b0;
      const RLD_GLOBAL uint16_t* xr = a.xa() + (size_t)(ok ? sm.rows[b0 + p * 16 + cl] : 0) * R;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const uint32_t k = ks * 32 + lg * 8;
        bop[p][ks] = (ok && k < R) ? load16(xr + k) : zero16();
      }
    }
  };
  auto load_base = [&](int b0, int cnt_, uint4 (&bv)[FV]) {
    const int nb = min(cnt_ - b0, kRows);
#pragma unroll
    for (int i = 0; i < FV; ++i) {
      const int rl = frow + 8 * i;
      bv[i] = (rl < nb && fcol_ok) ? load16(a.out() + (size_t)sm.rows[b0 + rl] * os + j0 + c8)
                                   : zero16();
    }
  };
  for (;;) {
    uint4 bop[PT][NKS], bv[FV];
    if (cnt > 0) {
      load_xa(0, cnt, bop);
      load_base(0, cnt, bv);
    }
    issue_point();
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        if (ks * 32 + lg * 8 >= (int)R) aop[m][ks] = zero16();
    // pass: MFMA (deltas to LDS), the next pass's xa goes out, the fold, the
    // next pass's base values go out
    for (int b0 = 0; b0 < cnt; b0 += kRows) {
      const int nb = min(cnt - b0, kRows);
      const bool more = b0 + kRows < cnt;
#pragma unroll
      for (int p = 0; p < PT; ++p) {
        if (p * 16 >= nb) break;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) acc = mfma_bf16_16x16x32(aop[m][ks], bop[p][ks], acc);
          // lane holds delta[row p*16+cl][cols m*16 + 4*lg .. +3] of this wave's slice
          *reinterpret_cast<uint2*>(&sm.dl[(p * 16 + cl) * kStride + wave * 64 + m * 16 + 4 * lg]) =
              make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
        }
      }
      if (more) load_xa(b0 + kRows, cnt, bop);
      issue_point();
      __syncthreads();
#pragma unroll
      for (int i = 0; i < FV; ++i) {
        const int rl = frow + 8 * i;
        if (rl < nb && fcol_ok) {
          const uint4 dv = *reinterpret_cast<const uint4*>(&sm.dl[rl * kStride + c8]);
          store16(a.out() + (size_t)sm.rows[b0 + rl] * os + j0 + c8, fold8(bv[i], dv, scale));
        }
      }
      if (more) load_base(b0 + kRows, cnt, bv);
      issue_point();
      __syncthreads();
    }
    if (pos >= n) break;
    cnt = collect_slot_rows(a.seq_slot(), n, &pos, s, sm.rows, sm.wcount, key0);
  }
}

// One-pass item: slot s, output columns [j0, j0 + 512) of route a.  With
// xa_writer it also stores the xa rows of s (column group 0 of each slot),
// with zero_writer the zero xa rows of rows that fold nothing.
__device__ void onepass_item(const BgmvArgs& a, int s, uint32_t j0, bool xa_writer,
                             bool zero_writer, OnePassSmem& sm) {
  constexpr int kStride = OnePassSmem::kStride;
  const uint32_t n = a.n, R = a.R, k_in = a.k_in, n_out = a.n_out, os = a.os;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lg = lane >> 4;
  const int cl = lane & 15;
  // every row's slot (n <= 1024) and the slot's table entries: one round
  const int key = threadIdx.x < n ? a.seq_slot()[threadIdx.x] : -1;
  const SlotEntry ent = slot_entry(a, s);
  if (zero_writer && threadIdx.x < n && !slot_active(a, key)) {
    for (uint32_t cc = 0; cc < R; cc += 8)
      store16(a.xa() + (size_t)threadIdx.x * R + cc, zero16());
  }
  if (!ent.active()) return;
  const int cnt = append_hits<kOpWaves>(key == s, threadIdx.x, sm.rows, 0, sm.wcount);
  if (cnt == 0) return;
  const RLD_GLOBAL uint16_t* A = gp<const uint16_t>(ent.a);
  const RLD_GLOBAL uint16_t* B = gp<const uint16_t>(ent.b);
  const float scale = ent.scale;

  // this wave's chunk c = wave: the shrink's wave w of that chunk owns steps
  // w + 4i (i < 4); a step is valid below the chunk's end
  const uint32_t c = (uint32_t)wave;
  const bool has_chunk = c < a.nch;
  const uint32_t kb = c * a.kc;
  const uint32_t ke = has_chunk ? min(kb + a.kc, k_in) : kb;
  const uint32_t nsteps = has_chunk ? (ke - kb + 31) / 32 : 0;
  // The chunk's A tile (rows 0..15 of A_s, the xa columns, clamped past
  // max_rank like the shrink) in the contiguous shape: load i takes rows 2i
  // and 2i + 1, a lane 16 bytes of one row's 512.  From L2 (the tile's later
  // readers are the slot's other column groups) this shape arrives about three
  // times faster than the MFMA fragments' 16 rows x 64 bytes; the tile goes
  // through this wave's LDS region into the fragments.
  uint4 araw[8];
  {
    const uint32_t kof = kb + (uint32_t)(lane & 31) * 8u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 2 * i + (lane >> 5);
      const RLD_GLOBAL uint16_t* ar = A + (size_t)(r < (int)R ? r : 0) * k_in;
      araw[i] = load16(kof < ke ? ar + kof : A);
    }
  }
  // B rows of this wave's 32 output columns as MFMA A operands (one K step:
  // max_rank <= 16 < 32), clamped like the expand
  uint4 aop[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const uint32_t col = j0 + wave * 32 + m * 16 + cl;
    const uint32_t k = lg * 8;
    aop[m] = load16((col < n_out && k < R) ? B + (size_t)col * R + k : B);
    if (k >= R) aop[m] = zero16();
  }
  // fold mapping: thread t folds row t / 64 of the batch, columns 8 (t % 64) ..
  const int frow = threadIdx.x >> 6;
  const int c8 = (threadIdx.x & 63) * 8;
  const bool fcol_ok = j0 + c8 < n_out;

  // x fragments of a batch's rows (row cl) for the chunk's steps; base values
  uint4 xf[8];
  uint4 bv;
  auto load_batch = [&](int b0) {
    const int nb = min(cnt - b0, 16);
    const bool ok = cl < nb;
    const RLD_GLOBAL uint16_t* xr = a.x() + (size_t)(ok ? sm.rows[b0 + cl] : 0) * a.xs;
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const uint32_t kof = kb + st * 32 + lg * 8;
      xf[st] = (ok && (uint32_t)st < nsteps && kof < ke) ? load16(xr + kof) : zero16();
    }
    bv = (frow < nb && fcol_ok) ? load16(a.out() + (size_t)sm.rows[b0 + frow] * os + j0 + c8)
                                : zero16();
  };
  load_batch(0);
  issue_point();
  // A fragments of the chunk's 8 steps from the staged tile (zero past the
  // chunk, as the shrink's masked steps); then every wave has its fragments and
  // the staging region is free for the wave sums and the delta tile
  uint4 af[8];
  {
    uint4* stg = sm.u.stage[wave];
#pragma unroll
    for (int i = 0; i < 8; ++i) stg[(2 * i + (lane >> 5)) * OnePassSmem::kStageRow + (lane & 31)] = araw[i];
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const uint32_t kof = kb + st * 32 + lg * 8;
      const bool ok = (uint32_t)st < nsteps && kof < ke;
      af[st] = ok ? stg[cl * OnePassSmem::kStageRow + st * 4 + lg] : zero16();
    }
  }
  __syncthreads();

  for (int b0 = 0; b0 < cnt; b0 += 16) {
    const int nb = min(cnt - b0, 16);
    if (b0 > 0) {
      load_batch(b0);
      issue_point();
    }
    // the shrink's four wave chains of chunk c and their wave-order sum
    floatx4 part = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int st = w + 4 * i;
        acc = mfma_bf16_16x16x32(st < 8 ? xf[st] : zero16(), st < 8 ? af[st] : zero16(), acc);
      }
      part = w == 0 ? acc : part + acc;
    }
    sm.u.w.red[wave][lane] = part;
    __syncthreads();
    // chunk sums in chunk order, rounded: xa[row 4g+i][col] of lane (g, col)
    if (threadIdx.x < 256) {
      const int l = threadIdx.x >> 2, i = threadIdx.x & 3;
      float sum = sm.u.w.red[0][l][i];
      for (uint32_t cc = 1; cc < a.nch; ++cc) sum = sum + sm.u.w.red[cc][l][i];
      const int row = 4 * (l >> 4) + i, col = l & 15;
      const uint16_t v = (uint16_t)f32_to_bf16(sum);
      sm.xs[row * 16 + col] = v;
      if (xa_writer && row < nb && (uint32_t)col < R)
        a.xa()[(size_t)sm.rows[b0 + row] * R + col] = v;
    }
    __syncthreads();
    // expand: xa of row cl, k = 8 lg .. (zero past max_rank)
    const uint4 bop = (uint32_t)(lg * 8) < R
                          ? *reinterpret_cast<const uint4*>(&sm.xs[cl * 16 + lg * 8])
                          : zero16();
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const floatx4 acc = mfma_bf16_16x16x32(aop[m], bop, floatx4{0.f, 0.f, 0.f, 0.f});
      // lane holds delta[row cl][cols m*16 + 4*lg .. +3] of this wave's slice
      *reinterpret_cast<uint2*>(&sm.u.w.dl[cl * kStride + wave * 32 + m * 16 + 4 * lg]) =
          make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
    }
    __syncthreads();
    if (frow < nb && fcol_ok) {
      const uint4 dv = *reinterpret_cast<const uint4*>(&sm.u.w.dl[frow * kStride + c8]);
      store16(a.out() + (size_t)sm.rows[b0 + frow] * os + j0 + c8, fold8(bv, dv, scale));
    }
    __syncthreads();
  }
}

template <int NT, int NW, int QTO = 0>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(QTO ? 6 : 1)))
void bgmv_shrink_kernel(BgmvArgs a, uint32_t total) {
  __shared__ ShrinkSmem<NT, NW, QTO> sm;
  // the column groups of one (slot, chunk) share an XCD, and so the x rows in
  // its L2
  const uint32_t w = xcd_group_item(a.ncg);
  if (w >= total) return;
  shrink_item<NT, NW, QTO>(a, w, sm);
}

// k split: xa[row, column] = bf16(sum over chunks, in chunk order, of the
// partials).  Base rows have zero partials (written by the shrink), so every
// row is handled alike and no routing is read.  One thread per xa element in
// one-wave blocks, so that the partials' reads spread over many CUs (a call's
// n*R elements are a few thousand at decode sizes); up to kReduceBatch chunk
// loads go out before their adds.
constexpr int kReduceBatch = 24;

// Thread t of a call's reduce: row t / R, column t % R.
__device__ __forceinline__ void reduce_unit(const BgmvArgs& a, uint32_t t) {
  const uint32_t row = t / a.R;
  const uint32_t col = t % a.R;
  const RLD_GLOBAL float* p = a.partial() + (size_t)row * a.R + col;
  const size_t cstride = (size_t)a.n * a.R;  // floats per chunk
  float sum = 0.f;
  for (uint32_t c0 = 0; c0 < a.nch; c0 += kReduceBatch) {
    float v[kReduceBatch];
#pragma unroll
    for (int j = 0; j < kReduceBatch; ++j) v[j] = p[(c0 + j < a.nch ? c0 + j : c0) * cstride];
    // every load of the batch goes out before the first add (no instruction
    // is scheduled across this point)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < kReduceBatch; ++j)
      if (c0 + j < a.nch) sum = (c0 + j == 0) ? v[j] : sum + v[j];
  }
  a.xa()[(size_t)row * a.R + col] = (uint16_t)f32_to_bf16(sum);
}

__global__ __launch_bounds__(kReduceThreads) void bgmv_reduce_kernel(BgmvArgs a) {
  const uint32_t t = blockIdx.x * kReduceThreads + threadIdx.x;
  if (t >= a.n * a.R) return;
  reduce_unit(a, t);
}

template <int NKS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NKS <= 2 ? (kLeanRows == 16 ? 6 : 5) : 4))) void bgmv_expand_lean_kernel(BgmvArgs a) {
  __shared__ ExpandLeanSmem sm;
  expand_lean_item<NKS>(a, (int)blockIdx.y, blockIdx.x * ExpandLeanSmem::kCols, sm);
}

template <int NKS, int MT>
__global__ __launch_bounds__(256) void bgmv_expand_kernel(BgmvArgs a) {
  __shared__ ExpandSmem<MT> sm;
  expand_item<NKS, MT>(a, (int)blockIdx.y, blockIdx.x * ExpandSmem<MT>::kCols, sm, blockIdx.z,
                       gridDim.z);
}

// Several routes over the same rows (rld_bgmv_multi): one launch of each
// kernel serves every route, the routes' items concatenated (route r: shrink
// items [first[r], first[r+1]), expand column tiles [tfirst[r], tfirst[r+1])).
// Each route's items are the single-route call's items, so its results are
// bit-identical to that call's.
constexpr uint32_t kMaxRoutes = 4;

struct BgmvMulti {
  BgmvArgs a[kMaxRoutes];
  uint32_t first[kMaxRoutes + 1];
  uint32_t tfirst[kMaxRoutes + 1];
  uint32_t nr;
};

__device__ __forceinline__ uint32_t route_of(const uint32_t* first, uint32_t nr, uint32_t w) {
  uint32_t r = 0;
  while (r + 1 < nr && w >= first[r + 1]) ++r;
  return r;
}

template <int NT, int NW>
__global__ __launch_bounds__(NW * kWave) void bgmv_shrink_multi_kernel(BgmvMulti m,
                                                                        uint32_t total) {
  __shared__ ShrinkSmem<NT, NW> sm;
  // every route has the same column groups: a group never spans two routes
  const uint32_t w = xcd_group_item(m.a[0].ncg);
  if (w >= total) return;
  const uint32_t r = route_of(m.first, m.nr, w);
  shrink_item<NT, NW>(m.a[r], w - m.first[r], sm);
}

__global__ __launch_bounds__(kReduceThreads) void bgmv_reduce_multi_kernel(BgmvMulti m) {
  const uint32_t per = m.a[0].n * m.a[0].R;  // n and R are shared
  const uint32_t t = blockIdx.x * kReduceThreads + threadIdx.x;
  const uint32_t r = t / per;
  if (r >= m.nr) return;
  reduce_unit(m.a[r], t - r * per);
}

template <int NKS, int MT>
__global__ __launch_bounds__(256) void bgmv_expand_multi_kernel(BgmvMulti m) {
  __shared__ ExpandSmem<MT> sm;
  const uint32_t r = route_of(m.tfirst, m.nr, blockIdx.x);
  if (blockIdx.y >= m.a[r].max_loras) return;
  expand_item<NKS, MT>(m.a[r], (int)blockIdx.y, (blockIdx.x - m.tfirst[r]) * ExpandSmem<MT>::kCols,
                       sm);
}

// Items of a one-pass launch: (route r, slot s, column group g), g fastest,
// so that a slot's groups are consecutive and land on one XCD.
__global__ __launch_bounds__(kOpThreads) void bgmv_onepass_kernel(BgmvMulti m, uint32_t total) {
  __shared__ OnePassSmem sm;
  const uint32_t w = xcd_work_item(total);
  if (w >= total) return;
  const uint32_t r = route_of(m.first, m.nr, w);
  const BgmvArgs& a = m.a[r];
  const uint32_t ng = (a.n_out + kOpCols - 1) / kOpCols;
  const uint32_t t = w - m.first[r];
  const int s = (int)(t / ng);
  const uint32_t g = t % ng;
  onepass_item(a, s, g * kOpCols, g == 0, g == 0 && (uint32_t)s == a.max_loras - 1, sm);
}

// Workspace: fp32 partials [nch][n][R] (k split only).
static size_t round16(size_t v) { return (v + 15) & ~(size_t)15; }

static size_t partial_bytes(uint32_t n, uint32_t k_in, uint32_t R) {
  const uint32_t nch = div_ceil(k_in, bgmv_chunk(k_in, R));
  return nch > 1 ? round16((size_t)nch * n * R * sizeof(float)) : 0;
}

static int make_args(const rld_route* route, const void* x, uint32_t x_row_stride,
                     const int32_t* seq_slot, uint32_t n, void* xa, void* workspace,
                     size_t workspace_bytes, void* base_out, uint32_t out_row_stride,
                     BgmvArgs* a) {
  *a = BgmvArgs{};
  const uint32_t R = route->max_rank, k_in = route->k_in;
  const size_t need = partial_bytes(n, k_in, R);
  if (need) {
    if (!workspace || workspace_bytes < need) return RLD_ENOSPACE;
    if (!aligned16(workspace)) return RLD_EALIGN;
  }
  char* ws = static_cast<char*>(workspace);
  a->x_ = reinterpret_cast<uint64_t>(x);
  a->seq_ = reinterpret_cast<uint64_t>(seq_slot);
  a->atab_ = reinterpret_cast<uint64_t>(route->a_table);
  a->btab_ = reinterpret_cast<uint64_t>(route->b_table);
  a->stab_ = reinterpret_cast<uint64_t>(route->scale_table);
  a->partial_ = reinterpret_cast<uint64_t>(ws);
  a->xa_ = reinterpret_cast<uint64_t>(xa);
  a->out_ = reinterpret_cast<uint64_t>(base_out);
  a->xs = x_row_stride;
  a->n = n;
  a->max_loras = route->max_loras;
  a->k_in = k_in;
  a->n_out = route->n_out;
  a->R = R;
  a->kc = bgmv_chunk(k_in, R);
  a->nch = div_ceil(k_in, a->kc);
  a->ncg = div_ceil(R, 16u * bgmv_nt(R));
  a->os = out_row_stride;
  return RLD_OK;
}

typedef void (*BgmvKernel)(BgmvArgs);

// A call's shrink items and chunk-reduce threads fit the 32-bit item indices
// and grids of its launches (with room for the grid's rounding up).
static bool launch_fits(uint64_t items, uint64_t reduce_threads) {
  return items <= (1ull << 30) && reduce_threads <= (1ull << 30);
}

// Expand items of 256 output columns (16*4 per wave).  (512-column items,
// half the blocks, measured slower on the decode FFN shapes.)
constexpr int kExpMT = 4;

static BgmvKernel pick_expand(uint32_t R) {
  switch (div_ceil(R, 32)) {
    case 1: return bgmv_expand_kernel<1, kExpMT>;
    case 2: return bgmv_expand_kernel<2, kExpMT>;
    case 3: return bgmv_expand_kernel<3, kExpMT>;
    default: return bgmv_expand_kernel<4, kExpMT>;
  }
}

typedef void (*BgmvMultiKernel)(BgmvMulti);

// The classic expand holds 168 registers a lane at max_rank 64, three blocks
// a CU: 768 resident on MI355X's 256 CUs.  A routed grid larger than that
// (the FFN decode shapes: 48 column tiles x 32 slots) takes the lean item,
// six blocks a CU, which runs the grid in one round; the results are the same
// bits either way.
constexpr uint32_t kClassicExpandResident = 768;

static BgmvKernel pick_expand_routed(uint32_t R, uint32_t tiles, uint32_t slots) {
  if ((uint64_t)tiles * slots <= kClassicExpandResident) return pick_expand(R);
  switch (div_ceil(R, 32)) {
    case 1: return bgmv_expand_lean_kernel<1>;
    case 2: return bgmv_expand_lean_kernel<2>;
    case 3: return bgmv_expand_lean_kernel<3>;
    default: return bgmv_expand_lean_kernel<4>;
  }
}

static BgmvMultiKernel pick_expand_multi(uint32_t R) {
  switch (div_ceil(R, 32)) {
    case 1: return bgmv_expand_multi_kernel<1, kExpMT>;
    case 2: return bgmv_expand_multi_kernel<2, kExpMT>;
    case 3: return bgmv_expand_multi_kernel<3, kExpMT>;
    default: return bgmv_expand_multi_kernel<4, kExpMT>;
  }
}

typedef void (*ShrinkKernel)(BgmvArgs, uint32_t);
typedef void (*ShrinkMultiKernel)(BgmvMulti, uint32_t);

// Routed eight-wave calls with k_in above 4096 (the FFN down projection: 1536
// items of 24 chunks) take 64-row batches and a two-subtile wave-sum round:
// 80 registers and 35 KB of LDS, three blocks a CU instead of two, so the
// items run in two rounds instead of three.  Batching does not enter a row's
// sums, so the results are the same bits.
static bool shrink_rows64(uint32_t k_in, uint32_t nt, uint32_t nw) {
  return nw == 8 && nt == 2 && k_in > 4096u;
}

// Shrink kernel of (column tiles per item, waves per block).
static ShrinkKernel pick_shrink(uint32_t nt, uint32_t nw, bool rows64 = false) {
  if (rows64) return bgmv_shrink_kernel<2, 8, 4>;
  if (nw == 8) return nt == 4 ? bgmv_shrink_kernel<4, 8> : bgmv_shrink_kernel<2, 8>;
  return nt == 1 ? bgmv_shrink_kernel<1, 4>
                 : (nt == 2 ? bgmv_shrink_kernel<2, 4> : bgmv_shrink_kernel<4, 4>);
}

static ShrinkMultiKernel pick_shrink_multi(uint32_t nt, uint32_t nw) {
  if (nw == 8) return bgmv_shrink_multi_kernel<2, 8>;
  return nt == 1 ? bgmv_shrink_multi_kernel<1, 4> : bgmv_shrink_multi_kernel<2, 4>;
}

static uint32_t onepass_items(const rld_route* route) {
  return div_ceil(route->n_out, (uint32_t)kOpCols) * route->max_loras;
}

// The one-pass fold serves calls whose k-split shrink has 256-wide chunks
// (at most sixteen) and four waves, over batches of at most kOpMaxRows rows,
// when its (slot, column group) items fit one round of one block per CU (each
// item reads its slot's whole A tile, so more items would mostly add reads);
// its results are those of the three launches, bit for bit, so the choice is
// free.
constexpr uint64_t kOpMaxItems = 256;

static bool use_onepass(const rld_route* const* routes, uint32_t nroutes, uint32_t n) {
  const uint32_t k_in = routes[0]->k_in, R = routes[0]->max_rank;
  if (!(R <= 16 && n <= (uint32_t)kOpMaxRows && k_in <= (uint32_t)(kOpWaves * kOpChunk) &&
        bgmv_chunk(k_in, R) <= (uint32_t)kOpChunk && bgmv_shrink_waves(k_in, R) == 4))
    return false;
  uint64_t items = 0;
  for (uint32_t r = 0; r < nroutes; ++r) items += onepass_items(routes[r]);
  return items <= kOpMaxItems;
}

}  // namespace rld

using namespace rld;

extern "C" size_t rld_bgmv_workspace_bytes(uint32_t n, uint32_t k_in, uint32_t max_rank,
                                           uint32_t max_loras) {
  if (k_in == 0 || max_rank == 0 || max_loras == 0) return 0;
  return partial_bytes(n, k_in, max_rank);
}

extern "C" int rld_bgmv_launches(const rld_route* const* routes, uint32_t nroutes, uint32_t n) {
  if (!routes || nroutes == 0 || nroutes > kMaxRoutes || n == 0) return 0;
  for (uint32_t r = 0; r < nroutes; ++r)
    if (check_route(routes[r]) != RLD_OK || routes[r]->k_in != routes[0]->k_in ||
        routes[r]->max_rank != routes[0]->max_rank)
      return 0;
  if (use_onepass(routes, nroutes, n)) return 1;
  return bgmv_chunk(routes[0]->k_in, routes[0]->max_rank) < routes[0]->k_in ? 3 : 2;
}

extern "C" int rld_bgmv_shrink(const rld_route* route, const void* x, uint32_t x_row_stride,
                               const int32_t* seq_slot, uint32_t n, void* xa, void* workspace,
                               size_t workspace_bytes, void* stream) {
  int st = check_route(route);
  if (st) return st;
  if (route->max_loras > 65535u) return RLD_EUNSUPPORTED;
  if (n == 0) return RLD_OK;
  if (!seq_slot || !xa) return RLD_EINVAL;
  if ((st = check_rows(x, x_row_stride, route->k_in))) return st;
  if (!aligned16(xa)) return RLD_EALIGN;
  BgmvArgs a;
  if ((st = make_args(route, x, x_row_stride, seq_slot, n, xa, workspace, workspace_bytes,
                      nullptr, 0, &a)))
    return st;
  if (!launch_fits((uint64_t)route->max_loras * a.nch * a.ncg, (uint64_t)n * a.R))
    return RLD_EUNSUPPORTED;
  const uint32_t total = route->max_loras * a.nch * a.ncg;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  const dim3 grid(xcd_group_grid(total, a.ncg));
  const uint32_t nw = bgmv_shrink_waves(a.k_in, a.R);
  hipLaunchKernelGGL(pick_shrink(bgmv_nt(a.R), nw, shrink_rows64(a.k_in, bgmv_nt(a.R), nw)),
                     grid, dim3(nw * kWave), 0, hs, a, total);
  if ((st = launch_status())) return st;
  if (a.nch > 1) {
    hipLaunchKernelGGL(bgmv_reduce_kernel, dim3(div_ceil(n * a.R, kReduceThreads)),
                       dim3(kReduceThreads), 0, hs, a);
    return launch_status();
  }
  return RLD_OK;
}

extern "C" int rld_bgmv_expand_fold(const rld_route* route, const void* xa,
                                    const int32_t* seq_slot, uint32_t n, void* base_out,
                                    uint32_t out_row_stride, void* stream) {
  int st = check_route(route);
  if (st) return st;
  if (route->max_loras > 65535u) return RLD_EUNSUPPORTED;
  if (n == 0) return RLD_OK;
  if (!seq_slot || !xa) return RLD_EINVAL;
  if (!aligned16(xa)) return RLD_EALIGN;
  if ((st = check_rows(base_out, out_row_stride, route->n_out))) return st;
  BgmvArgs a = {};
  a.seq_ = reinterpret_cast<uint64_t>(seq_slot);
  a.atab_ = reinterpret_cast<uint64_t>(route->a_table);
  a.btab_ = reinterpret_cast<uint64_t>(route->b_table);
  a.stab_ = reinterpret_cast<uint64_t>(route->scale_table);
  a.xa_ = reinterpret_cast<uint64_t>(xa);
  a.out_ = reinterpret_cast<uint64_t>(base_out);
  a.n = n;
  a.max_loras = route->max_loras;
  a.k_in = route->k_in;
  a.n_out = route->n_out;
  a.R = route->max_rank;
  a.os = out_row_stride;
  const uint32_t tiles = div_ceil(route->n_out, 64u * kExpMT);
  static_assert(ExpandLeanSmem::kCols == 64 * kExpMT, "both expands take 256-column tiles");
  // the classic item splits a slot's rows of a batch over four items (grid z)
  // once a slot can hold more than one 64-row batch
  const bool classic = (uint64_t)tiles * route->max_loras <= kClassicExpandResident;
  const uint32_t zc = classic && n > (uint32_t)kExpRows ? 4u : 1u;
  hipLaunchKernelGGL(pick_expand_routed(a.R, tiles, route->max_loras),
                     dim3(tiles, route->max_loras, zc), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), a);
  return launch_status();
}

extern "C" int rld_bgmv(const rld_route* route, const void* x, uint32_t x_row_stride,
                        const int32_t* seq_slot, uint32_t n, void* base_out,
                        uint32_t out_row_stride, void* xa, void* workspace,
                        size_t workspace_bytes, void* stream) {
  int st = check_route(route);
  if (st) return st;
  if (n == 0) return RLD_OK;
  if ((st = check_rows(base_out, out_row_stride, route->n_out))) return st;
  if (use_onepass(&route, 1, n)) {
    // the checks of the two stages, then one launch
    if (route->max_loras > 65535u) return RLD_EUNSUPPORTED;
    if (!seq_slot || !xa) return RLD_EINVAL;
    if ((st = check_rows(x, x_row_stride, route->k_in))) return st;
    if (!aligned16(xa)) return RLD_EALIGN;
    BgmvMulti m = {};
    m.nr = 1;
    if ((st = make_args(route, x, x_row_stride, seq_slot, n, xa, workspace, workspace_bytes,
                        base_out, out_row_stride, &m.a[0])))
      return st;
    const uint32_t items = onepass_items(route);
    m.first[1] = items;
    hipLaunchKernelGGL(bgmv_onepass_kernel, dim3(xcd_grid(items)), dim3(kOpThreads), 0,
                       reinterpret_cast<hipStream_t>(stream), m, items);
    return launch_status();
  }
  st = rld_bgmv_shrink(route, x, x_row_stride, seq_slot, n, xa, workspace, workspace_bytes,
                       stream);
  if (st) return st;
  return rld_bgmv_expand_fold(route, xa, seq_slot, n, base_out, out_row_stride, stream);
}

extern "C" size_t rld_bgmv_multi_workspace_bytes(uint32_t n, uint32_t k_in, uint32_t max_rank,
                                                 uint32_t nroutes) {
  if (k_in == 0 || max_rank == 0 || nroutes == 0) return 0;
  return (size_t)nroutes * partial_bytes(n, k_in, max_rank);
}

extern "C" int rld_bgmv_multi(const rld_route* const* routes, uint32_t nroutes, const void* x,
                              uint32_t x_row_stride, const int32_t* seq_slot, uint32_t n,
                              void* const* base_out, const uint32_t* out_row_stride,
                              void* const* xa, void* workspace, size_t workspace_bytes,
                              void* stream) {
  if (!routes || nroutes == 0 || !base_out || !out_row_stride || !xa) return RLD_EINVAL;
  if (nroutes > kMaxRoutes) return RLD_EUNSUPPORTED;
  int st;
  for (uint32_t r = 0; r < nroutes; ++r) {
    if ((st = check_route(routes[r]))) return st;
    if (routes[r]->max_loras > 65535u) return RLD_EUNSUPPORTED;
    if (routes[r]->k_in != routes[0]->k_in || routes[r]->max_rank != routes[0]->max_rank)
      return RLD_EINVAL;
  }
  if (n == 0) return RLD_OK;
  const uint32_t k_in = routes[0]->k_in, R = routes[0]->max_rank;
  if (!seq_slot) return RLD_EINVAL;
  if ((st = check_rows(x, x_row_stride, k_in))) return st;
  for (uint32_t r = 0; r < nroutes; ++r) {
    if (!xa[r]) return RLD_EINVAL;
    if (!aligned16(xa[r])) return RLD_EALIGN;
    if ((st = check_rows(base_out[r], out_row_stride[r], routes[r]->n_out))) return st;
  }
  const size_t pb = partial_bytes(n, k_in, R);
  if (pb) {
    if (!workspace || workspace_bytes < nroutes * pb) return RLD_ENOSPACE;
    if (!aligned16(workspace)) return RLD_EALIGN;
  }
  {
    uint64_t all = 0;
    for (uint32_t r = 0; r < nroutes; ++r)
      all += (uint64_t)routes[r]->max_loras * div_ceil(k_in, bgmv_chunk(k_in, R)) *
             div_ceil(R, 16u * bgmv_nt(R));
    if (!launch_fits(all, (uint64_t)nroutes * n * R)) return RLD_EUNSUPPORTED;
  }
  BgmvMulti m = {};
  m.nr = nroutes;
  uint32_t items = 0, tiles = 0, slots = 0;
  for (uint32_t r = 0; r < nroutes; ++r) {
    // each route's partials in its own part of the workspace
    void* ws = pb ? static_cast<char*>(workspace) + r * pb : nullptr;
    if ((st = make_args(routes[r], x, x_row_stride, seq_slot, n, xa[r], ws, pb, base_out[r],
                        out_row_stride[r], &m.a[r])))
      return st;
    m.first[r] = items;
    items += routes[r]->max_loras * m.a[r].nch * m.a[r].ncg;
    m.tfirst[r] = tiles;
    tiles += div_ceil(routes[r]->n_out, 64u * kExpMT);
    slots = max(slots, routes[r]->max_loras);
  }
  m.first[nroutes] = items;
  m.tfirst[nroutes] = tiles;
  if (tiles > 0x7fffffffu) return RLD_EUNSUPPORTED;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (use_onepass(routes, nroutes, n)) {
    uint32_t op = 0;
    for (uint32_t r = 0; r < nroutes; ++r) {
      m.first[r] = op;
      op += onepass_items(routes[r]);
    }
    m.first[nroutes] = op;
    hipLaunchKernelGGL(bgmv_onepass_kernel, dim3(xcd_grid(op)), dim3(kOpThreads), 0, hs, m, op);
    return launch_status();
  }
  const dim3 grid(xcd_group_grid(items, m.a[0].ncg));
  const uint32_t nw = bgmv_shrink_waves(k_in, R);
  hipLaunchKernelGGL(pick_shrink_multi(bgmv_nt(R), nw), grid, dim3(nw * kWave), 0, hs, m, items);
  if ((st = launch_status())) return st;
  if (m.a[0].nch > 1) {
    hipLaunchKernelGGL(bgmv_reduce_multi_kernel,
                       dim3(div_ceil(nroutes * n * R, kReduceThreads)),
                       dim3(kReduceThreads), 0, hs, m);
    if ((st = launch_status())) return st;
  }
  hipLaunchKernelGGL(pick_expand_multi(R), dim3(tiles, slots), dim3(256), 0, hs, m);
  return launch_status();
}

// ------------------------------------------------------------ unrouted ----

static int check_pair(const rld_pair* p) {
  if (!p || !p->a || !p->b) return RLD_EINVAL;
  int st = check_dims(p->k_in, p->n_out, p->max_rank);
  if (st) return st;
  if (!aligned16(p->a) || !aligned16(p->b)) return RLD_EALIGN;
  return RLD_OK;
}

static void dense_args(const rld_pair* pair, uint32_t m, BgmvArgs* a) {
  *a = BgmvArgs{};
  a->dense = 1;
  a->a_dense = reinterpret_cast<uint64_t>(pair->a);
  a->b_dense = reinterpret_cast<uint64_t>(pair->b);
  a->scale_dense = pair->scale;
  a->n = m;
  a->max_loras = 1;
  a->k_in = pair->k_in;
  a->n_out = pair->n_out;
  a->R = pair->max_rank;
  a->kc = bgmv_chunk(pair->k_in, pair->max_rank);
  a->nch = div_ceil(pair->k_in, a->kc);
  a->ncg = div_ceil(pair->max_rank, 16u * bgmv_nt(pair->max_rank, true));
}

extern "C" size_t rld_lora_workspace_bytes(uint32_t m, uint32_t k_in, uint32_t max_rank) {
  if (k_in == 0 || max_rank == 0) return 0;
  return partial_bytes(m, k_in, max_rank);
}

extern "C" int rld_lora_shrink(const rld_pair* pair, const void* x, uint32_t x_row_stride,
                               uint32_t m, void* xa, void* workspace, size_t workspace_bytes,
                               void* stream) {
  int st = check_pair(pair);
  if (st) return st;
  if (m == 0) return RLD_OK;
  if (!xa) return RLD_EINVAL;
  if ((st = check_rows(x, x_row_stride, pair->k_in))) return st;
  if (!aligned16(xa)) return RLD_EALIGN;
  const size_t need = partial_bytes(m, pair->k_in, pair->max_rank);
  if (need) {
    if (!workspace || workspace_bytes < need) return RLD_ENOSPACE;
    if (!aligned16(workspace)) return RLD_EALIGN;
  }
  BgmvArgs a;
  dense_args(pair, m, &a);
  a.x_ = reinterpret_cast<uint64_t>(x);
  a.xs = x_row_stride;
  a.xa_ = reinterpret_cast<uint64_t>(xa);
  a.partial_ = reinterpret_cast<uint64_t>(workspace);
  // the routed calls' wave rule, so a row's sums are added in the same order
  const uint32_t nw = bgmv_shrink_waves(a.k_in, a.R);
  const uint32_t tile = (uint32_t)dense_shrink_rows((int)nw);
  if (!launch_fits((uint64_t)div_ceil(m, tile) * a.nch * a.ncg, (uint64_t)m * a.R))
    return RLD_EUNSUPPORTED;
  const uint32_t total = div_ceil(m, tile) * a.nch * a.ncg;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  const dim3 grid(xcd_group_grid(total, a.ncg));
  hipLaunchKernelGGL(pick_shrink(bgmv_nt(a.R, true), nw), grid, dim3(nw * kWave), 0, hs, a,
                     total);
  if ((st = launch_status())) return st;
  if (a.nch > 1) {
    hipLaunchKernelGGL(bgmv_reduce_kernel, dim3(div_ceil(m * a.R, kReduceThreads)),
                       dim3(kReduceThreads), 0, hs, a);
    return launch_status();
  }
  return RLD_OK;
}

extern "C" int rld_lora_expand_fold(const rld_pair* pair, const void* xa, uint32_t m,
                                    void* base_out, uint32_t out_row_stride, void* stream) {
  int st = check_pair(pair);
  if (st) return st;
  if (m == 0) return RLD_OK;
  if (!xa) return RLD_EINVAL;
  if (!aligned16(xa)) return RLD_EALIGN;
  if ((st = check_rows(base_out, out_row_stride, pair->n_out))) return st;
  const uint32_t tiles = div_ceil(m, (uint32_t)kDenseExpandRows);
  if (tiles > 65535u) return RLD_EUNSUPPORTED;
  BgmvArgs a;
  dense_args(pair, m, &a);
  a.xa_ = reinterpret_cast<uint64_t>(xa);
  a.out_ = reinterpret_cast<uint64_t>(base_out);
  a.os = out_row_stride;
  hipLaunchKernelGGL(pick_expand(a.R), dim3(div_ceil(pair->n_out, 64 * kExpMT), tiles), dim3(256),
                     0, reinterpret_cast<hipStream_t>(stream), a);
  return launch_status();
}

extern "C" int rld_lora_delta(const rld_pair* pair, const void* x, uint32_t x_row_stride,
                              uint32_t m, void* base_out, uint32_t out_row_stride, void* xa,
                              void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_pair(pair);
  if (st) return st;
  if (m == 0) return RLD_OK;
  if ((st = check_rows(base_out, out_row_stride, pair->n_out))) return st;
  if (div_ceil(m, (uint32_t)kDenseExpandRows) > 65535u) return RLD_EUNSUPPORTED;
  st = rld_lora_shrink(pair, x, x_row_stride, m, xa, workspace, workspace_bytes, stream);
  if (st) return st;
  return rld_lora_expand_fold(pair, xa, m, base_out, out_row_stride, stream);
}

// ------------------------------------------------------- no allocation ----
//
// rld_bgmv for callers that cannot allocate (code under HIP graph capture,
// serving loops that forbid hipMalloc): the xa arena and the k-split partials
// live in this file-scope device array instead of caller buffers.  Each GPU the
// library runs on holds its own copy until the process ends.  Its device
// address is taken once per device (hipGetSymbolAddress, with that device
// current) and kept; kernels get that address as an argument, never the
// array's name, which in host code is only a stand-in for the symbol.

static __device__ __align__(256) unsigned char scratch[RLD_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

// Device address of `scratch` on the current device (looked up on the first
// call made with that device current), or an error status.
static int scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    record_hip_error(e);
    return RLD_ELAUNCH;
  }
  if (dev < 0 || dev >= kMaxDevices) return RLD_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      record_hip_error(e != hipSuccess ? e : hipErrorInvalidSymbol);
      return RLD_ELAUNCH;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return RLD_OK;
}

static size_t noalloc_xa_bytes(uint32_t n, uint32_t R) {
  return ((size_t)n * R * 2 + 255) & ~(size_t)255;
}

extern "C" int rld_bgmv_noalloc(const rld_route* route, const void* x, uint32_t x_row_stride,
                                const int32_t* seq_slot, uint32_t n, void* base_out,
                                uint32_t out_row_stride, void* stream) {
  int st = check_route(route);
  if (st) return st;
  if (n == 0) return RLD_OK;
  if ((st = check_rows(base_out, out_row_stride, route->n_out))) return st;
  if ((st = check_rows(x, x_row_stride, route->k_in))) return st;
  if (!seq_slot) return RLD_EINVAL;
  // every size check before the device is touched
  const size_t xab = noalloc_xa_bytes(n, route->max_rank);
  const size_t pb = partial_bytes(n, route->k_in, route->max_rank);
  if (xab + pb > (size_t)RLD_NOALLOC_SCRATCH_BYTES) return RLD_ENOSPACE;
  void* sp = nullptr;
  if ((st = scratch_on_current_device(&sp))) return st;
  char* xa = static_cast<char*>(sp);
  char* ws = pb ? xa + xab : nullptr;
  return rld_bgmv(route, x, x_row_stride, seq_slot, n, base_out, out_row_stride, xa, ws, pb,
                  stream);
}
