// Tile geometry and every index computation of the fused attention kernels.
//
// All address arithmetic of the fused kernels goes through the functions in
// this header, which compile for the host as well as the device, so a CPU
// test can enumerate every thread, tile and fragment of a launch and check
// that each global and LDS access stays inside its buffer before a kernel is
// ever run.
//
// Work split (the query-block split of FlashAttention-2 that "Flash
// attention in PyTorch, then in Triton" uses, section "A kernel in Triton"):
// one workgroup of 4 wave64s owns kBlockM = 128 consecutive query rows of
// one (batch, head) slice; each wave owns 32 of them and walks the key tiles
// in ascending order.
//
// MFMA orientation. The score tile is computed transposed, S^T = K * Q^T, on
// 32x32 MFMAs: the A operand is a K fragment (row = key), the B operand a Q
// fragment (column = query). An MFMA accumulator register r of lane l holds
// row 8*(r/4) + 4*(l/32) + (r%4), column l%32, so every lane owns ONE query
// (l % 32) and 16 of the 32 keys of a 32x32 tile; the other 16 keys of that
// query sit in lane l ^ 32. Row max and row sum are in-lane reductions plus
// one exchange between the two 32-lane halves. The output is accumulated
// transposed the same way, O^T = V^T * P^T, so the per-query rescale factor
// is a per-lane scalar.
//
// K-index freedom. An MFMA pairs slot s of lane-half h of its A operand with
// slot s of lane-half h of its B operand for the same reduction index, so any
// assignment of reduction indices to (half, slot) works as long as A and B
// use the same one. The P fragment inherits its key order from the
// accumulator layout; the fragments read from the K and V tiles follow it.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define ATTN_HD __host__ __device__ inline
#else
#define ATTN_HD inline
#endif

namespace attn {

constexpr int kHeadDim = 64;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBlockM = 32 * kWaves;  // query rows per workgroup

// ---- 16-bit (bf16 / f16) path -------------------------------------------
constexpr int kBlockN16 = 64;     // keys per LDS tile

// ---- fp32 path -----------------------------------------------------------
constexpr int kBlockN32 = 32;
constexpr int kKStride32 = 68;    // floats per K row: 64 + 4 pad
constexpr int kVStride32 = 36;    // floats per V^T row: 32 + 4 pad
constexpr int kKTile32 = kBlockN32 * kKStride32;
constexpr int kVTile32 = kHeadDim * kVStride32;

static_assert(kKStride32 % 4 == 0 && kVStride32 % 4 == 0,
              "fp32 LDS rows must stay 16-byte aligned");
static_assert(2 * 4 * (kKTile32 + kVTile32) <= 64 * 1024,
              "fp32 double-buffered K and V^T tiles must fit 64 KiB");

// Row (key or head-dim index) held by accumulator register r of a lane in
// lane-half h of a 32x32 MFMA output tile.
ATTN_HD int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// Workgroup -> (slice bh, query tile qt). Workgroups are dealt round-robin
// to the 8 XCDs, so when the count divides by 8 the consecutive logical tiles
// are regrouped to land on one XCD: each XCD walks whole (batch, head)
// slices, and the slice's K and V stay in that XCD's L2. Causal launches
// take the heaviest (last) query tile of a slice first.
ATTN_HD void tile_of(int block, int total, int nq, bool causal, int* bh,
                     int* qt) {
    int L = block;
    if ((total & 7) == 0) {
        const int per = total >> 3;
        L = (block & 7) * per + (block >> 3);
    }
    *bh = L / nq;
    const int t = L - *bh * nq;
    *qt = causal ? nq - 1 - t : t;
}

// Number of key tiles of `bn` keys query tile qt (of bm rows) reads: every
// tile that holds a key visible to one of its valid rows (rows < T).
ATTN_HD int key_tiles(int qt, int T, int bn, bool causal, int bm = kBlockM) {
    const int all = (T + bn - 1) / bn;
    if (!causal) return all;
    int last = qt * bm + bm - 1;
    if (last > T - 1) last = T - 1;
    const int n = last / bn + 1;
    return n < all ? n : all;
}

// Number of leading key tiles that need no mask for any row of query tile
// qt: every key of the tile is < T and (causal) <= the tile's first row.
// Tiles from here to key_tiles() are the edge tiles (diagonal or ragged).
ATTN_HD int main_tiles(int qt, int T, int bn, bool causal, int bm = kBlockM) {
    int n = T / bn;  // tiles wholly below T
    if (causal) {
        const int c = (qt * bm + 1) / bn;  // tiles with k0 + bn - 1 <= q0
        if (c < n) n = c;
    }
    const int all = key_tiles(qt, T, bn, causal, bm);
    return n < all ? n : all;
}

// ---- 16-bit direct-to-LDS staging ---------------------------------------------
// K and V tiles (64 keys x 64 dims, 128-byte rows, no padding) are written by
// global_load_lds_dwordx4: lane l of a wave instruction lands its 16 bytes at
// LDS base + 16*l, so a wave instruction fills 8 consecutive rows and each
// lane fetches whichever global 16-byte chunk belongs in its slot. Chunks are
// XOR-swizzled within a row so the fragment reads hit distinct banks:
//   K: chunk c of row r sits at slot c ^ ((r >> 1) & 7)   (16-byte reads by
//      16 consecutive rows at one chunk),
//   V: chunk c of row r sits at slot c ^ ((r & 2) << 1)   (8-byte transposed
//      reads of 4 consecutive rows x 4 chunks per 16 lanes).
constexpr int kTileBytes16 = kBlockN16 * kHeadDim * 2;   // 8 KiB per K or V tile
ATTN_HD int swz_k(int row) { return (row >> 1) & 7; }
ATTN_HD int swz_v(int row) { return (row & 2) << 1; }
// Byte offset of (row, 16-byte chunk) of a K tile / of element (row, d) of a
// V tile inside their 8 KiB tiles.
ATTN_HD int k_byte(int row, int chunk) { return row * 128 + ((chunk ^ swz_k(row)) << 4); }
ATTN_HD int v_byte(int row, int d) {
    return row * 128 + (((d >> 3) ^ swz_v(row)) << 4) + ((d & 7) << 1);
}
// Direct load: wave w's instruction i (0, 1) of a tile, lane l: the tile row
// and logical chunk this lane fetches (it lands at byte 1024*(2w+i) + 16*l).
ATTN_HD void dl_src(int w, int i, int l, bool is_v, int* row, int* chunk) {
    const int slot = (2 * w + i) * 64 + l;
    *row = slot >> 3;
    *chunk = (slot & 7) ^ (is_v ? swz_v(*row) : swz_k(*row));
}
// Load schedule of the 16-bit kernel. K tiles and V tiles have rings of
// their own: K tile t in stage t % 4, V tile t in stage t % 4. Batch u is
// what the iteration u issues after its barrier: K(u + 3) and V(u + 2), each
// when it exists (0 <= tile < n); the prologue issues batches -3, -2, -1,
// i.e. K(0), then K(1) and V(0), then K(2) and V(1). Main iteration j
// (weights of tile j, S(j+1) = K(j+1) Q^T, O += V(j-1) P(j-1), and in the
// rare rescale case S(j) again from K(j)) reads K(j), K(j+1) and V(j-1), all
// in batch j - 2 or older, so before its barrier a wave waits until only
// batch j - 1 is in flight. The reloads of batch j go to K stage (j+3) % 4
// (K(j-1), last read in iteration j - 1) and V stage (j+2) % 4 (V(j-2), read
// in iteration j-1), both finished by every wave at iteration j's barrier.
// The edge tiles that follow (at most two, the last ones) find their K and V
// loaded: their batches are empty.
ATTN_HD int batch_k(int u, int n) { return (u + 3 >= 0 && u + 3 < n) ? u + 3 : -1; }
ATTN_HD int batch_v(int u, int n) { return (u + 2 >= 0 && u + 2 < n) ? u + 2 : -1; }
// load instructions per wave in batch u (2 per K or V tile)
ATTN_HD int batch_size(int u, int n) {
    return 2 * (batch_k(u, n) >= 0) + 2 * (batch_v(u, n) >= 0);
}
constexpr int kRingK = 4;
constexpr int kRingV = 4;

// K fragment of S^T tile nt, step ks for lane (ql, h): 16 bytes, dims
// 16ks + 8h .. +7 of key 32nt + ql.
ATTN_HD int kfrag_byte(int ql, int h, int nt, int ks) {
    return k_byte(32 * nt + ql, 2 * ks + h);
}
// V^T fragment for the O^T tile mt, step ks, from two ds_read_b64_tr_b16
// (half 0: slots 0-3, half 1: slots 4-7). Within each 16-lane group the
// transposed read hands lane i element (i % 4) of the 8-byte chunks read by
// lanes 4r + i/4, r = 0..3. So lane l addresses row 16ks + 8*half + 4h + r,
// dims d0 + 4c .. +3 (r = (l%16)/4, c = l%4, d0 = 32mt + 16((l/16)%2),
// h = l/32), and receives V[16ks + 8*half + 4h + 0..3][32mt + l%32]: the keys
// the P fragment holds in those slots, at its head dimension.
ATTN_HD int vtr_byte(int l, int mt, int ks, int half) {
    const int j = l & 15, r = j >> 2, c = j & 3;
    const int g = (l >> 4) & 1, h = l >> 5;
    return v_byte(16 * ks + 8 * half + 4 * h + r, 32 * mt + 16 * g + 4 * c);
}
// Both swizzles depend on the lane alone (bits 1..3 of the key row for K,
// bit 1 for V), so a lane keeps one LDS address per K step ks and per V
// half-tile mt and reaches the rest by constant offsets:
//   kfrag_byte(ql, h, nt, ks)     = kfrag_byte(ql, h, 0, ks) + kKfragNtStride * nt
//   vtr_byte(l, mt, ks, half)     = vtr_byte(l, mt, 0, 0) + kVtrKsStride * ks
//                                   + kVtrHalfStride * half
constexpr int kKfragNtStride = 32 * 128;
constexpr int kVtrKsStride = 16 * 128;
constexpr int kVtrHalfStride = 8 * 128;
// Byte offset, within a K or V tile in global memory (64 rows of 128 B), of
// the 16 bytes that direct load i of lane l of wave w fetches.
ATTN_HD int dl_global_byte(int w, int i, int l, bool is_v) {
    int row, chunk;
    dl_src(w, i, l, is_v, &row, &chunk);
    return row * kHeadDim * 2 + chunk * 16;
}

// ---- 16-bit forward, eight-wave workgroups (D = 64) --------------------------
// kWaves8 wave64s own 32 query rows each (kBlockM8 = 256 per workgroup) and
// share every K and V tile: one 1 KiB direct load per wave per tile (wave w
// is the 4-wave schedule's instruction w: tile rows 8w .. 8w + 7), K tile t
// in stage t % kRing8 of its ring, V likewise, tiles issued kAhead8 ahead.
// Each wave runs the plain loop (S, weights, P.V of one tile at a time); at
// <= 128 VGPRs two workgroups put four waves on every SIMD, whose matrix and
// vector work the hardware interleaves.
constexpr int kWaves8 = 8;
constexpr int kThreads8 = 64 * kWaves8;
constexpr int kBlockM8 = 32 * kWaves8;
constexpr int kRing8 = 4;
constexpr int kAhead8 = kRing8 - 1;
// Tiles of query tile qt that wave w computes (a key visible to one of its
// valid rows), and how many leading ones need no mask (every key < T and,
// causal, <= the wave's first row). The wave's tiles between the two (at
// most its diagonal tile and the ragged last tile) take the masked step.
// A wave whose rows all lie past T computes none.
ATTN_HD int w8_seen(int qt, int w, int T, bool causal, int bm = kBlockM8) {
    const int wq0 = qt * bm + 32 * w;
    if (wq0 >= T) return 0;
    const int all = (T + kBlockN16 - 1) / kBlockN16;
    if (!causal) return all;
    const int last = wq0 + 31 < T - 1 ? wq0 + 31 : T - 1;
    const int n = last / kBlockN16 + 1;
    return n < all ? n : all;
}
ATTN_HD int w8_main(int qt, int w, int T, bool causal, int bm = kBlockM8) {
    const int wq0 = qt * bm + 32 * w;
    if (wq0 >= T) return 0;
    int n = T / kBlockN16;
    if (causal) {
        const int c = (wq0 + 1) / kBlockN16;
        if (c < n) n = c;
    }
    const int seen = w8_seen(qt, w, T, causal, bm);
    return n < seen ? n : seen;
}
// Workgroup -> (slice, 256-row query tile) of the eight-wave kernel. As in
// tile_of, each XCD keeps whole slices (their K and V stay in its L2), but
// within an XCD the order is query tile major: the heaviest causal tiles
// of all its slices first, then the next ones. With 256-row tiles a slice
// has half as many tiles of twice the work, and walking slice by slice
// leaves the last heavy tiles of the last slice to run alone at the end.
ATTN_HD void tile_of8(int block, int total, int nq, bool causal, int* bh, int* qt) {
    const int BH = total / nq;
    if ((total & 7) != 0 || (BH & 7) != 0) {
        tile_of(block, total, nq, causal, bh, qt);
        return;
    }
    const int spx = BH >> 3;  // slices per XCD
    const int x = block & 7, i = block >> 3;
    *bh = x * spx + i % spx;
    const int t = i / spx;
    *qt = causal ? nq - 1 - t : t;
}
// Which 16-bit D = 64 forward a call runs.
//  - The eight-wave kernel (256-row workgroups, K and V tiles shared by the
//    most rows) on full calls whose grid has at least one workgroup per CU,
//    and on causal calls whose heaviest query tile (4 nq key tiles, nq =
//    ceil(T / 256)) is at most 7/4 of the work per workgroup slot (two per
//    CU, 512 slots): 4 nq <= 7/4 * BH * 2 nq (nq + 1) / 512, that is
//    BH (nq + 1) >= 585. Below that the heaviest tiles' key loops set the
//    call's time (measured: the eight-wave kernel ahead by 5% at BH (nq + 1)
//    = 640 and 816, behind by 2-28% from 544 down).
//  - Otherwise its key-split form: kSplit8 groups of waves share the query
//    rows (kBlockM8s = 128 per workgroup, twice the workgroups), group g
//    computes the key tiles t with t % kSplit8 == g, and the groups'
//    partial results merge through LDS at the end, so the heaviest tile
//    runs half as many tiles in turn. Every causal call that does not take
//    the eight-wave kernel takes this one; full calls take it while its
//    grid has at most one workgroup per CU (kW8MinGrid).
//  - Otherwise (full calls between the two) the 128-row kernel.
constexpr int kW8MinGrid = 256;
constexpr int kW8CausalWork = 600;
constexpr int kSplit8 = 2;
constexpr int kBlockM8s = kBlockM8 / kSplit8;
ATTN_HD bool fwd16_eight_waves(long long BH, int T, bool causal) {
    const long long nq = (T + kBlockM8 - 1) / kBlockM8;
    return causal ? BH * (nq + 1) >= kW8CausalWork : nq * BH >= kW8MinGrid;
}
ATTN_HD bool fwd16_key_split(long long BH, int T, bool causal) {
    if (fwd16_eight_waves(BH, T, causal)) return false;
    return causal || (long long)((T + kBlockM8s - 1) / kBlockM8s) * BH <= kW8MinGrid;
}

// ---- other head dimensions (16-bit forward, D = 32 or 128) -----------------
// Tiles of 64 keys x D dims, rows of 2D bytes (C = D / 8 chunks of 16 B),
// filled by direct loads of 1 KiB wave instructions (D / 8 per tile, D / 32
// per wave). Swizzles, per D, keeping the row fragment reads (16 rows at one
// chunk per quarter-wave) and the transposed reads (4 rows x 4 columns per
// 16 lanes, 32 lanes per phase) free of bank conflicts:
//   D = 128 (16 chunks, every row starts at bank 0): K chunk c of row r at
//     c ^ (r & 15); V chunk c at c ^ (4 * (r & 3)) (the 4 rows of a
//     transposed read land in distinct quarters of the row);
//   D = 32 (4 chunks, 4 rows per 256 bytes): K chunk c at c ^ ((r >> 2) & 3);
//     V needs none (a transposed read's 4 rows x 4 chunks are 256 whole
//     bytes);
//   D = 64: swz_k and swz_v above, so that HeadDim<64> addresses the tiles
//     of the D = 64 kernels byte for byte (the decode kernels take every
//     head dimension through this struct).
template <int D>
struct HeadDim {
    static_assert(D == 32 || D == 64 || D == 128, "head dimension without a layout");
    static constexpr int kChunks = D / 8;
    static constexpr int kRowBytes = 2 * D;
    static constexpr int kTileBytes = 64 * kRowBytes;
    static constexpr int kInstr = kTileBytes / 1024;      // wave instructions per tile
    static constexpr int kInstrPerWave = kInstr / kWaves;
    static constexpr int kSteps = D / 16;                  // MFMA reduction steps of S
    static constexpr int kOTiles = D / 32;                 // 32-dim tiles of O
    ATTN_HD static int swz_k(int r) {
        return D == 128 ? (r & 15) : D == 64 ? attn::swz_k(r) : ((r >> 2) & 3);
    }
    ATTN_HD static int swz_v(int r) {
        return D == 128 ? 4 * (r & 3) : D == 64 ? attn::swz_v(r) : 0;
    }
    ATTN_HD static int k_byte(int row, int chunk) {
        return row * kRowBytes + ((chunk ^ swz_k(row)) << 4);
    }
    ATTN_HD static int v_byte(int row, int d) {
        return row * kRowBytes + (((d >> 3) ^ swz_v(row)) << 4) + ((d & 7) << 1);
    }
    // direct load: instruction i of a tile (0 .. kInstr-1), lane l
    ATTN_HD static void src(int i, int l, bool is_v, int* row, int* chunk) {
        const int slot = i * 64 + l;
        *row = slot / kChunks;
        const int c = slot % kChunks;
        *chunk = c ^ (is_v ? swz_v(*row) : swz_k(*row));
    }
    ATTN_HD static int global_byte(int i, int l, bool is_v) {
        int row, chunk;
        src(i, l, is_v, &row, &chunk);
        return row * kRowBytes + chunk * 16;
    }
    // K fragment of S^T tile nt, step ks, lane (ql, h); nt adds 32 rows
    ATTN_HD static int kfrag(int ql, int h, int nt, int ks) {
        return k_byte(32 * nt + ql, 2 * ks + h);
    }
    // transposed V^T fragment read (8 bytes) of O^T tile mt, step ks, half;
    // ks adds 16 rows and half 8 rows; mt needs a lane base
    ATTN_HD static int vtr(int l, int mt, int ks, int half) {
        const int j = l & 15, r = j >> 2, c = j & 3;
        const int g = (l >> 4) & 1, h = l >> 5;
        return v_byte(16 * ks + 8 * half + 4 * h + r, 32 * mt + 16 * g + 4 * c);
    }
    // Q fragment columns of lane-half h, step ks
    ATTN_HD static int q_col(int h, int ks) { return 16 * ks + 8 * h; }
};

// ---- backward pass (16-bit) -----------------------------------------------
// The backward kernels read some 64-row tiles both ways: row fragments
// (16 consecutive rows at one 16-byte chunk per quarter-wave, as the K tile
// of the forward) and transposed fragments (4 rows x 4 columns per 16 lanes,
// as the V tile of the forward). One swizzle serves both without bank
// conflicts: chunk c of row r sits at slot c ^ swz_b(r), where
//   swz_b(r) = (((r >> 1) & 1) << 2) | ((r >> 2) & 3)
// is a bijection of bits 1..3 of the row (16 consecutive rows of one parity
// land on 8 distinct slots) and flips slot bit 2 between rows r and r + 2 of
// a group of four (the two halves of a transposed read's row quad land on
// disjoint slots).
// The backward's row workspace: -delta of every row, then lse * log2(e) of
// every row, each array starting on a 256-byte boundary (this many floats
// apart).
ATTN_HD long long bwd_ws_stride(long long rows) { return (rows + 63) / 64 * 64; }
constexpr int kBwdBlockKV = 128;  // keys per workgroup of the dK/dV kernel
constexpr int kBwdBlockQ = 64;    // queries per tile it streams
ATTN_HD int swz_b(int row) { return (((row >> 1) & 1) << 2) | ((row >> 2) & 3); }
ATTN_HD int b_byte(int row, int chunk) { return row * 128 + ((chunk ^ swz_b(row)) << 4); }
ATTN_HD int b_elem_byte(int row, int d) {
    return row * 128 + (((d >> 3) ^ swz_b(row)) << 4) + ((d & 7) << 1);
}
// Direct load of a backward tile: wave w's instruction i (0, 1), lane l ->
// tile row and logical chunk (it lands at byte 1024*(2w+i) + 16*l).
ATTN_HD void dlb_src(int w, int i, int l, int* row, int* chunk) {
    const int slot = (2 * w + i) * 64 + l;
    *row = slot >> 3;
    *chunk = (slot & 7) ^ swz_b(*row);
}
ATTN_HD int dlb_global_byte(int w, int i, int l) {
    int row, chunk;
    dlb_src(w, i, l, &row, &chunk);
    return row * kHeadDim * 2 + chunk * 16;
}
// Row fragment (A operand: 32 rows of tile half mt, reduction step ks over
// the 64 columns) of lane (ql, h): 16 bytes, columns 16ks + 8h .. +7 of row
// 32mt + ql. The row half mt adds 4096 bytes; the step needs a lane base.
ATTN_HD int bfrag_byte(int ql, int h, int mt, int ks) {
    return b_byte(32 * mt + ql, 2 * ks + h);
}
// Transposed fragment (A operand: columns 32ct .. +31 as rows, reduction over
// 16 tile rows per step ks) read by lane l as two 8-byte transposing reads
// (half 0, 1): the same lane pattern as the forward's V tile, in swz_b. The
// step ks adds 2048 bytes; (ct, half) need a lane base each.
ATTN_HD int btr_byte(int l, int ct, int ks, int half) {
    const int j = l & 15, r = j >> 2, c = j & 3;
    const int g = (l >> 4) & 1, h = l >> 5;
    return b_elem_byte(16 * ks + 8 * half + 4 * h + r, 32 * ct + 16 * g + 4 * c);
}
constexpr int kBfragMtStride = 32 * 128;
constexpr int kBtrKsStride = 16 * 128;
// Workgroup -> (slice bh, key block kb) of the dK/dV kernel: XCD-grouped like
// tile_of; causal launches take the heaviest (first) key blocks first, as
// key block kb is seen by the queries from kb * kBwdBlockKV on.
ATTN_HD void bwd_kv_tile_of(int block, int total, int nkb, bool causal, int* bh, int* kb) {
    int L = block;
    if ((total & 7) == 0) {
        const int per = total >> 3;
        L = (block & 7) * per + (block >> 3);
    }
    *bh = L / nkb;
    const int t = L - *bh * nkb;
    *kb = causal ? t : nkb - 1 - t;
}
// First query tile (of kBwdBlockQ) that sees any key of key block kb.
ATTN_HD int bwd_first_qtile(int kb, bool causal) {
    return causal ? (kb * kBwdBlockKV) / kBwdBlockQ : 0;
}
// Wave w of the dK/dV kernel's key block kb (keys kb * kBwdBlockKV + 32w ..
// + 31) and query tile u counted from bwd_first_qtile: the first u the wave
// sees (causal: a tile whose last query comes before the wave's first key
// is skipped), and whether tile u needs masks (a query before one of the
// wave's keys, or rows past T).
ATTN_HD int bwd_kv_first_seen(int kb, int w, int n, bool causal) {
    const int kw0 = kb * kBwdBlockKV + 32 * w;
    const int t0 = bwd_first_qtile(kb, causal);
    int u = 0;
    if (causal)
        while (u < n && (t0 + u) * kBwdBlockQ + kBwdBlockQ - 1 < kw0) ++u;
    return u;
}
ATTN_HD bool bwd_kv_edge(int kb, int w, int u, int T, bool causal) {
    const int kw0 = kb * kBwdBlockKV + 32 * w;
    const int q0 = (bwd_first_qtile(kb, causal) + u) * kBwdBlockQ;
    return (causal && q0 < kw0 + 31) || q0 + kBwdBlockQ > T;
}
// The single-kernel backward (dQ added with atomics) shares the dK/dV
// kernel's work map and adds two LDS tiles holding dS^T of the workgroup's
// key block for the current query tile (row = key, column = query, swz_b).
// Wave w writes rows 32w .. 32w + 31 (tile w / 2); lane (ql, h) of half mt
// writes its 4 packed values of register group g, queries 32mt + 8g + 4h ..
// + 3 of key 32w + ql, as one 8-byte store.
ATTN_HD int bwd_ds_byte(int w, int ql, int h, int mt, int g) {
    return kTileBytes16 * (w >> 1) + b_elem_byte(32 * (w & 1) + ql, 32 * mt + 8 * g + 4 * h);
}
// Its dQ product: wave w owns the 32 x 32 output block of queries
// 32 * bwd_dq_qhalf(w) .. and dims 32 * bwd_dq_dhalf(w) .. of the tile,
// summed over the block's 128 keys.
ATTN_HD int bwd_dq_qhalf(int w) { return w >> 1; }
ATTN_HD int bwd_dq_dhalf(int w) { return w & 1; }
// Wave w of the dQ kernel's query tile qt (queries qt * kBlockM + 32w ..
// + 31) and key tile u of kBlockN16 keys: how many key tiles the wave sees
// (causal: none past its last query), and whether tile u needs masks (a key
// after one of the wave's queries, or keys past T).
ATTN_HD int bwd_q_tiles_seen(int qt, int w, int n, bool causal) {
    const int wq0 = qt * kBlockM + 32 * w;
    if (!causal) return n;
    const int last = (wq0 + 31) / kBlockN16 + 1;
    return last < n ? last : n;
}
ATTN_HD bool bwd_q_edge(int qt, int w, int u, int T, bool causal) {
    const int wq0 = qt * kBlockM + 32 * w;
    const int k0 = u * kBlockN16;
    return (causal && k0 + kBlockN16 - 1 > wq0) || k0 + kBlockN16 > T;
}

// ---- decode (few queries against a key/value cache) -------------------------
// A workgroup takes one tile of kDecTile queries and one chunk of keys; its 4
// waves take every fourth 32-key tile of the chunk. The chunk is chosen so
// that all workgroups run in one round, at most one per CU (256), a
// multiple of 4 waves x 32 keys: a workgroup's fixed start-up latency is
// paid once, and no CU carries two workgroups while others carry one
// (measured at 4 x 12 heads, one query, 8192 keys: 240 workgroups 27.6 us,
// 480 29.1 us, 288 33.0 us).
constexpr int kDecTile = 32;                             // keys per tile, queries per tile
constexpr int kDecTileBytes = kDecTile * kHeadDim * 2;   // 4 KiB at D = 64
// A 32-key tile of head dimension D is the first half of HeadDim<D>'s
// 64-key tile: same swizzles, D / 16 direct-load wave instructions.
template <int D>
constexpr int dec_tile_bytes() { return kDecTile * HeadDim<D>::kRowBytes; }
template <int D>
constexpr int dec_instr() { return dec_tile_bytes<D>() / 1024; }
ATTN_HD void decode_plan(int BH, int Tq, int Tk, int* nsplit, int* chunk) {
    const int nqt = (Tq + kDecTile - 1) / kDecTile;
    const long long base = (long long)BH * nqt;
    long long want = 256 / base;
    const int max_split = (Tk + kWaves * kDecTile - 1) / (kWaves * kDecTile);
    if (want > max_split) want = max_split;
    if (want < 1) want = 1;
    int ch = (int)((Tk + want - 1) / want);
    ch = (ch + kWaves * kDecTile - 1) / (kWaves * kDecTile) * (kWaves * kDecTile);
    *chunk = ch;
    *nsplit = (Tk + ch - 1) / ch;
}

// Q fragment of lane-half h for reduction step ks: dims 16*ks + 8*h .. +7.
ATTN_HD int q_col16(int h, int ks) { return 16 * ks + 8 * h; }

// ---- fp32 forward for small grids -----------------------------------------
// With fewer 128-row workgroups than CUs (one head of a few thousand tokens),
// the fp32 forward splits the keys inside a workgroup instead: kSplitWaves
// waves share 32 query rows, wave w takes key tiles w, w + kSplitWaves, ...
// and stages them in LDS of its own, and the waves' partial (O, m, l) merge
// through LDS at the end.
constexpr int kSplitWaves = 8;
constexpr int kSplitThreads = 64 * kSplitWaves;
constexpr int kSplitRows = 32;         // query rows per workgroup
constexpr int kSplitMinGrid = 256;     // 128-row workgroups below which it is used
constexpr int kSplitTileFloats = kKTile32 + kVTile32;   // one wave's K and V^T tile
constexpr int kMergeStride32 = 65;     // floats per row of a wave's partial O
ATTN_HD bool fwd32_split(long long BH, int T) {
    return (long long)((T + kBlockM - 1) / kBlockM) * BH < kSplitMinGrid;
}
static_assert(kSplitWaves * kSplitTileFloats * 4 <= 160 * 1024,
              "the split kernel's per-wave tiles must fit the LDS");
static_assert(kSplitWaves * kSplitRows * (kMergeStride32 + 2) <= kSplitWaves * kSplitTileFloats,
              "the merge area must fit in the tiles' LDS");

// ---- fp32 staging ----------------------------------------------------------
// K tile: 32 keys x 64 dims = 512 chunks of 16 B; chunks t and t + 256.
ATTN_HD void k_stage32(int t, int i, int* row, int* col) {
    const int c = t + kThreads * i;
    *row = c >> 4;
    *col = (c & 15) * 4;
}
ATTN_HD int k_lds32(int row, int col) { return row * kKStride32 + col; }
// V tile: keys key0, key0 + 1 at dims dim0 .. dim0 + 3, written transposed
// as one 64-bit pair per dim.
ATTN_HD void v_stage32(int t, int* key0, int* dim0) {
    *key0 = 2 * (t & 15);
    *dim0 = 4 * (t >> 4);
}
ATTN_HD int v_lds32(int dim, int key) { return dim * kVStride32 + key; }
// Q fragment of lane-half h, group g: dims 8*g + 4*h .. +3 (one MFMA step
// per dim, two steps' worth of dims per lane pair).
ATTN_HD int q_col32(int h, int g) { return 8 * g + 4 * h; }
ATTN_HD int kfrag32(int ql, int h, int g) {
    return ql * kKStride32 + 8 * g + 4 * h;
}
ATTN_HD int vfrag32(int ql, int h, int mt, int g) {
    return (32 * mt + ql) * kVStride32 + 8 * g + 4 * h;
}

}  // namespace attn
