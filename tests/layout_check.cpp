// CPU check of every index the fused kernels form, through the same
// functions the kernels call (online_softmax_amd/csrc/fused_layout.h):
//  - global loads/stores stay inside [B*H*T*D] (and lse inside [B*H*T]);
//  - LDS reads/writes stay inside their tiles and keep 16/8/4-byte alignment;
//  - each LDS stage writes every tile element exactly once (no stale reads);
//  - workgroup -> (slice, query tile) is a bijection;
//  - the key tiles a query tile walks cover every key its rows can see;
//  - the P fragment and the V^T fragment pair the same key in every
//    (lane, slot) of every PV step, and the K and Q fragments the same dim.
// Exit status 0 = all good; otherwise the first failure is printed.
#include <cstdio>
#include <cstdlib>
#include <set>
#include <algorithm>
#include <vector>

#include "fused_layout.h"

using namespace attn;

static int failures = 0;
#define CHECK(cond, ...)                                   \
    do {                                                   \
        if (!(cond)) {                                     \
            if (failures++ < 10) {                         \
                std::printf("FAIL %s:%d: ", __FILE__, __LINE__); \
                std::printf(__VA_ARGS__);                  \
                std::printf("\n");                         \
            }                                              \
        }                                                  \
    } while (0)

static void check_tile_map(int BH, int T, bool causal) {
    const int nq = (T + kBlockM - 1) / kBlockM;
    const int total = nq * BH;
    std::vector<int> seen((size_t)total, 0);
    for (int b = 0; b < total; ++b) {
        int bh, qt;
        tile_of(b, total, nq, causal, &bh, &qt);
        CHECK(bh >= 0 && bh < BH && qt >= 0 && qt < nq, "tile_of(%d) out of range", b);
        if (bh >= 0 && bh < BH && qt >= 0 && qt < nq) seen[(size_t)bh * nq + qt]++;
    }
    for (int i = 0; i < total; ++i) CHECK(seen[i] == 1, "tile %d hit %d times", i, seen[i]);
}

static void check_key_cover(int T, int bn, bool causal) {
    const int nq = (T + kBlockM - 1) / kBlockM;
    for (int qt = 0; qt < nq; ++qt) {
        const int n = key_tiles(qt, T, bn, causal);
        CHECK(n >= 1, "no key tile for qt %d", qt);
        int last_row = qt * kBlockM + kBlockM - 1;
        if (last_row > T - 1) last_row = T - 1;
        const int need = causal ? last_row : T - 1;  // last key any row sees
        CHECK((long)n * bn > need, "qt %d: %d tiles miss key %d", qt, n, need);
        CHECK((long)(n - 1) * bn <= need, "qt %d: tile %d sees nothing", qt, n - 1);
        CHECK((long)(n - 1) * bn < T, "qt %d: tile past T", qt);
        const int nm = main_tiles(qt, T, bn, causal);
        CHECK(nm >= 0 && nm <= n, "qt %d: main tiles %d of %d", qt, nm, n);
        // the pipelined 16-bit loop stages K two tiles ahead: edge tiles
        // (which stage only V) must be the last two at most
        if (bn == kBlockN16) CHECK(n - nm <= 2, "qt %d: %d edge tiles", qt, n - nm);
        for (int kt = 0; kt < nm; ++kt) {  // a main tile needs no mask at all
            CHECK((long)kt * bn + bn <= T, "qt %d: main tile %d ragged", qt, kt);
            if (causal)
                CHECK((long)kt * bn + bn - 1 <= (long)qt * kBlockM,
                      "qt %d: main tile %d crosses the diagonal", qt, kt);
        }
        // the first edge tile does need a mask for some row (or is ragged)
        if (nm < n) {
            const long k0 = (long)nm * bn;
            const bool ragged = k0 + bn > T;
            const bool diag = causal && k0 + bn - 1 > (long)qt * kBlockM;
            CHECK(ragged || diag, "qt %d: tile %d is edge without a reason", qt, nm);
        }
    }
}

// Global accesses of every 16-bit workgroup: the direct loads of every key
// tile it reads (full tiles: the slice buffer at the tile's offset plus the
// lane's offset; the ragged tile: rows clamped to T-1), its Q and O rows and
// lse; and the Q and O dims of every lane.
static void check16(int BH, int T, bool causal) {
    const long tensor = (long)BH * T * kHeadDim;  // elements
    const long slice_bytes = (long)T * kHeadDim * 2;
    const int nq = (T + kBlockM - 1) / kBlockM;
    const int total = nq * BH;
    for (int b = 0; b < total; ++b) {
        int bh, qt;
        tile_of(b, total, nq, causal, &bh, &qt);
        const long base = (long)bh * T * kHeadDim;
        const int n = key_tiles(qt, T, kBlockN16, causal);
        for (int kt = 0; kt < n; ++kt) {
            const long k0 = (long)kt * kBlockN16;
            for (int w = 0; w < kWaves; ++w)
                for (int i = 0; i < 2; ++i)
                    for (int l = 0; l < 64; ++l)
                        for (int is_v = 0; is_v < 2; ++is_v) {
                            const long voff = dl_global_byte(w, i, l, is_v);
                            long off;  // byte offset in the slice buffer
                            if (k0 + kBlockN16 <= T) {
                                off = k0 * kHeadDim * 2 + voff;
                            } else {
                                long r = k0 + (voff >> 7);
                                if (r > T - 1) r = T - 1;
                                off = r * kHeadDim * 2 + (voff & 127);
                            }
                            CHECK(off >= 0 && off + 16 <= slice_bytes && off % 16 == 0,
                                  "direct load outside the slice: wg %d tile %d wave %d lane %d",
                                  b, kt, w, l);
                            CHECK(base + off / 2 + 8 <= tensor, "direct load outside the tensor");
                        }
        }
        for (int t = 0; t < kThreads; ++t) {
            const int my_q = qt * kBlockM + 32 * (t >> 6) + (t & 31);
            if (my_q < T) {
                const long row = base + (long)my_q * kHeadDim;
                CHECK(row + kHeadDim <= tensor, "Q/O row");
                CHECK((long)bh * T + my_q < (long)BH * T, "lse");
            }
        }
    }
    for (int lane = 0; lane < 64; ++lane) {
        const int hh = lane >> 5;
        for (int ks = 0; ks < 4; ++ks) {
            const int qc = q_col16(hh, ks);
            CHECK(qc % 8 == 0 && qc + 8 <= kHeadDim, "q_col16");
        }
        for (int mt = 0; mt < 2; ++mt)
            for (int g = 0; g < 4; ++g) {
                const int d = 32 * mt + acc_row(4 * g, hh);
                CHECK(d % 4 == 0 && d + 4 <= kHeadDim, "O store dims");
            }
    }
}

static void check32(int BH, int T, bool causal) {
    const long tensor = (long)BH * T * kHeadDim;
    const int nq = (T + kBlockM - 1) / kBlockM;
    std::vector<int> kcov(kKTile32, 0), vcov(kVTile32, 0);
    for (int t = 0; t < kThreads; ++t) {
        for (int i = 0; i < 2; ++i) {
            int row, col;
            k_stage32(t, i, &row, &col);
            const int a = k_lds32(row, col);
            CHECK(row < kBlockN32 && col + 4 <= kHeadDim, "k_stage32");
            CHECK(a % 4 == 0 && a + 4 <= kKTile32, "k_lds32");
            for (int x = 0; x < 4; ++x) kcov[a + x]++;
        }
        int key0, dim0;
        v_stage32(t, &key0, &dim0);
        CHECK(key0 % 2 == 0 && key0 + 2 <= kBlockN32 && dim0 + 4 <= kHeadDim, "v_stage32");
        for (int j = 0; j < 4; ++j) {
            const int a = v_lds32(dim0 + j, key0);
            CHECK(a % 2 == 0 && a + 2 <= kVTile32, "v_lds32");
            vcov[a]++;
            vcov[a + 1]++;
        }
    }
    for (int r = 0; r < kBlockN32; ++r)
        for (int c = 0; c < kHeadDim; ++c) CHECK(kcov[k_lds32(r, c)] == 1, "K32 coverage");
    for (int d = 0; d < kHeadDim; ++d)
        for (int key = 0; key < kBlockN32; ++key)
            CHECK(vcov[v_lds32(d, key)] == 1, "V32 coverage");
    for (int lane = 0; lane < 64; ++lane) {
        const int ql = lane & 31, hh = lane >> 5;
        for (int g = 0; g < 8; ++g) {
            const int a = kfrag32(ql, hh, g);
            CHECK(a % 4 == 0 && a + 4 <= kKTile32, "kfrag32");
            CHECK(a == k_lds32(ql, q_col32(hh, g)), "K/Q dim pairing 32");
        }
        for (int mt = 0; mt < 2; ++mt)
            for (int g = 0; g < 4; ++g) {
                const int a = vfrag32(ql, hh, mt, g);
                CHECK(a % 4 == 0 && a + 4 <= kVTile32, "vfrag32");
                for (int i = 0; i < 4; ++i)  // PV step 4g+i uses register 4g+i
                    CHECK(a + i == v_lds32(32 * mt + ql, acc_row(4 * g + i, hh)),
                          "P/V key mismatch (fp32)");
            }
    }
    const int total = nq * BH;
    for (int b = 0; b < total; ++b) {
        int bh, qt;
        tile_of(b, total, nq, causal, &bh, &qt);
        const long base = (long)bh * T * kHeadDim;
        const int n = key_tiles(qt, T, kBlockN32, causal);
        for (int kt = 0; kt < n; ++kt) {
            const int k0 = kt * kBlockN32;
            for (int t = 0; t < kThreads; ++t) {
                for (int i = 0; i < 2; ++i) {
                    int row, col;
                    k_stage32(t, i, &row, &col);
                    if (k0 + row < T) {
                        const long a = base + (long)(k0 + row) * kHeadDim + col;
                        CHECK(a + 4 <= tensor && a % 4 == 0, "K32 global");
                    }
                }
                int key0, dim0;
                v_stage32(t, &key0, &dim0);
                for (int e = 0; e < 2; ++e)
                    if (k0 + key0 + e < T) {
                        const long a = base + (long)(k0 + key0 + e) * kHeadDim + dim0;
                        CHECK(a + 4 <= tensor && a % 4 == 0, "V32 global");
                    }
            }
        }
    }
}

// Direct-load staging and fragment reads of the 16-bit kernel: every chunk of
// a tile is fetched exactly once per stage; K fragments decode to the rows and
// dims they claim; the transposed V reads, simulated with the hardware rule
// (within 16 lanes, lane i receives element i%4 of the chunks of lanes
// 4r + i/4), hand every lane and slot the key the P fragment holds there at
// the lane's head dimension; and 16 consecutive-lane groups hit distinct
// 4-byte banks (64 banks).
static void decode_k(int byte, int* row, int* dim) {
    *row = byte / 128;
    const int slot = (byte % 128) / 16;
    *dim = ((slot ^ swz_k(*row)) * 8) + (byte % 16) / 2;
}
static void decode_v(int byte, int* row, int* dim) {
    *row = byte / 128;
    const int slot = (byte % 128) / 16;
    *dim = ((slot ^ swz_v(*row)) * 8) + (byte % 16) / 2;
}
static void check_direct16() {
    for (int is_v = 0; is_v < 2; ++is_v) {
        std::vector<int> cov(64 * 8, 0);
        for (int w = 0; w < kWaves; ++w)
            for (int i = 0; i < 2; ++i)
                for (int l = 0; l < 64; ++l) {
                    int row, chunk;
                    dl_src(w, i, l, is_v, &row, &chunk);
                    CHECK(row >= 0 && row < 64 && chunk >= 0 && chunk < 8, "dl_src range");
                    CHECK(dl_global_byte(w, i, l, is_v) == row * 128 + chunk * 16,
                          "direct load source offset");
                    const int dst = 1024 * (2 * w + i) + 16 * l;
                    const int want = is_v ? v_byte(row, 8 * chunk) : k_byte(row, chunk);
                    CHECK(dst == want, "direct load lands at the wrong slot");
                    cov[row * 8 + chunk]++;
                }
        for (int x = 0; x < 64 * 8; ++x) CHECK(cov[x] == 1, "tile chunk fetched %d times", cov[x]);
    }
    for (int nt = 0; nt < 2; ++nt)
        for (int ks = 0; ks < 4; ++ks) {
            std::vector<int> bank_use(64, 0);
            for (int l = 0; l < 64; ++l) {
                const int ql = l & 31, h = l >> 5;
                const int b = kfrag_byte(ql, h, nt, ks);
                CHECK(b % 16 == 0 && b + 16 <= kTileBytes16, "kfrag range");
                CHECK(b == kfrag_byte(ql, h, 0, ks) + kKfragNtStride * nt, "kfrag stride");
                int row, dim;
                decode_k(b, &row, &dim);
                CHECK(row == 32 * nt + ql && dim == 16 * ks + 8 * h, "K fragment decode");
            }
            for (int grp = 0; grp < 4; ++grp) {  // 16 lanes x 16 B = 256 B per cycle
                std::vector<int> used(64, 0);
                for (int l = 16 * grp; l < 16 * grp + 16; ++l) {
                    const int b = kfrag_byte(l & 31, l >> 5, nt, ks);
                    for (int x = 0; x < 4; ++x) used[(b / 4 + x) % 64]++;
                }
                for (int x = 0; x < 64; ++x) CHECK(used[x] <= 1, "K read bank conflict");
            }
        }
    for (int mt = 0; mt < 2; ++mt)
        for (int ks = 0; ks < 4; ++ks)
            for (int half = 0; half < 2; ++half) {
                int addr[64];
                for (int l = 0; l < 64; ++l) {
                    addr[l] = vtr_byte(l, mt, ks, half);
                    CHECK(addr[l] % 8 == 0 && addr[l] + 8 <= kTileBytes16, "vtr range");
                    CHECK(addr[l] == vtr_byte(l, mt, 0, 0) + kVtrKsStride * ks +
                                         kVtrHalfStride * half,
                          "vtr stride");
                }
                for (int l = 0; l < 64; ++l) {
                    const int g0 = l & ~15, i = l & 15;
                    const int ql = l & 31, h = l >> 5;
                    for (int r = 0; r < 4; ++r) {
                        const int src = g0 + 4 * r + i / 4;
                        int row, dim;
                        decode_v(addr[src] + 2 * (i % 4), &row, &dim);
                        const int slot = 4 * half + r;
                        // key of P slot `slot` at step ks, lane-half h
                        const int nt = ks >> 1, reg = (ks & 1) * 8 + slot;
                        const int pkey = 32 * nt + acc_row(reg, h);
                        CHECK(row == pkey && dim == 32 * mt + ql,
                              "V tr lane %d slot %d: row %d dim %d, want %d %d", l, slot, row,
                              dim, pkey, 32 * mt + ql);
                    }
                }
                for (int half32 = 0; half32 < 2; ++half32) {  // 32 lanes x 8 B per cycle
                    std::vector<int> used(64, 0);
                    for (int l = 32 * half32; l < 32 * half32 + 32; ++l)
                        for (int x = 0; x < 2; ++x) used[(addr[l] / 4 + x) % 64]++;
                    for (int x = 0; x < 64; ++x) CHECK(used[x] <= 1, "V tr read bank conflict");
                }
            }
}

// The backward tiles in swz_b: direct-load coverage, row fragments (decode,
// strides, bank conflicts), and transposed fragments simulated with the
// hardware rule, which must hand lane (column, half h) slot s of step ks the
// row the P / dS fragments hold there: 16ks + 8(s/4) + 4h + s%4.
static void decode_b(int byte, int* row, int* dim) {
    *row = byte / 128;
    const int slot = (byte % 128) / 16;
    *dim = ((slot ^ swz_b(*row)) * 8) + (byte % 16) / 2;
}
static void check_bwd_layout() {
    std::vector<int> cov(64 * 8, 0);
    for (int w = 0; w < kWaves; ++w)
        for (int i = 0; i < 2; ++i)
            for (int l = 0; l < 64; ++l) {
                int row, chunk;
                dlb_src(w, i, l, &row, &chunk);
                CHECK(row >= 0 && row < 64 && chunk >= 0 && chunk < 8, "dlb_src range");
                CHECK(1024 * (2 * w + i) + 16 * l == b_byte(row, chunk), "bwd direct load slot");
                CHECK(dlb_global_byte(w, i, l) == row * 128 + chunk * 16, "bwd load offset");
                cov[row * 8 + chunk]++;
            }
    for (int x = 0; x < 64 * 8; ++x) CHECK(cov[x] == 1, "bwd tile chunk fetched %d times", cov[x]);
    for (int mt = 0; mt < 2; ++mt)
        for (int ks = 0; ks < 4; ++ks) {
            for (int l = 0; l < 64; ++l) {
                const int ql = l & 31, h = l >> 5;
                const int b = bfrag_byte(ql, h, mt, ks);
                CHECK(b % 16 == 0 && b + 16 <= kTileBytes16, "bfrag range");
                CHECK(b == bfrag_byte(ql, h, 0, ks) + kBfragMtStride * mt, "bfrag stride");
                int row, dim;
                decode_b(b, &row, &dim);
                CHECK(row == 32 * mt + ql && dim == 16 * ks + 8 * h, "bwd row fragment decode");
            }
            for (int grp = 0; grp < 4; ++grp) {
                std::vector<int> used(64, 0);
                for (int l = 16 * grp; l < 16 * grp + 16; ++l) {
                    const int b = bfrag_byte(l & 31, l >> 5, mt, ks);
                    for (int x = 0; x < 4; ++x) used[(b / 4 + x) % 64]++;
                }
                for (int x = 0; x < 64; ++x) CHECK(used[x] <= 1, "bwd row read bank conflict");
            }
        }
    for (int ct = 0; ct < 2; ++ct)
        for (int ks = 0; ks < 4; ++ks)
            for (int half = 0; half < 2; ++half) {
                int addr[64];
                for (int l = 0; l < 64; ++l) {
                    addr[l] = btr_byte(l, ct, ks, half);
                    CHECK(addr[l] % 8 == 0 && addr[l] + 8 <= kTileBytes16, "btr range");
                    CHECK(addr[l] == btr_byte(l, ct, 0, half) + kBtrKsStride * ks, "btr stride");
                }
                for (int l = 0; l < 64; ++l) {
                    const int g0 = l & ~15, i = l & 15, h = l >> 5;
                    for (int r = 0; r < 4; ++r) {
                        const int src = g0 + 4 * r + i / 4;
                        int row, dim;
                        decode_b(addr[src] + 2 * (i % 4), &row, &dim);
                        const int s = 4 * half + r;
                        const int want_row = 16 * ks + 8 * (s / 4) + 4 * h + s % 4;
                        // the P / dS packing of step ks holds accumulator
                        // register 8(ks&1) + s of half-tile ks>>1
                        const int pk = 32 * (ks >> 1) + acc_row(8 * (ks & 1) + s, h);
                        CHECK(want_row == pk, "bwd packing order");
                        CHECK(row == want_row && dim == 32 * ct + (l & 31),
                              "bwd tr lane %d slot %d: row %d dim %d", l, s, row, dim);
                    }
                }
                for (int half32 = 0; half32 < 2; ++half32) {
                    std::vector<int> used(64, 0);
                    for (int l = 32 * half32; l < 32 * half32 + 32; ++l)
                        for (int x = 0; x < 2; ++x) used[(addr[l] / 4 + x) % 64]++;
                    for (int x = 0; x < 64; ++x) CHECK(used[x] <= 1, "bwd tr read bank conflict");
                }
            }
}

// The dK/dV kernel's work map: every (slice, key block) exactly once, and the
// first query tile it streams holds the first query that sees its first key.
static void check_bwd_map(int BH, int T, bool causal) {
    const int nkb = (T + kBwdBlockKV - 1) / kBwdBlockKV;
    const int nqt = (T + kBwdBlockQ - 1) / kBwdBlockQ;
    const int total = nkb * BH;
    std::vector<int> seen((size_t)total, 0);
    for (int b = 0; b < total; ++b) {
        int bh, kb;
        bwd_kv_tile_of(b, total, nkb, causal, &bh, &kb);
        CHECK(bh >= 0 && bh < BH && kb >= 0 && kb < nkb, "bwd_kv_tile_of range");
        if (bh >= 0 && bh < BH && kb >= 0 && kb < nkb) seen[(size_t)bh * nkb + kb]++;
        const int t0 = bwd_first_qtile(kb, causal);
        CHECK(t0 >= 0 && t0 < nqt, "first query tile %d of %d", t0, nqt);
        if (causal) {
            CHECK((long)t0 * kBwdBlockQ <= (long)kb * kBwdBlockKV, "first tile starts late");
            CHECK((long)(t0 + 1) * kBwdBlockQ > (long)kb * kBwdBlockKV, "first tile sees nothing");
        }
    }
    for (int i = 0; i < total; ++i) CHECK(seen[i] == 1, "key block %d hit %d times", i, seen[i]);
}

// Global accesses of the backward kernels: the tile loads of every
// workgroup (rows clamped to T-1 in a ragged tile), the lse/delta loads,
// and the rows each lane reads into registers and writes.
static void check_bwd_access(int BH, int T, bool causal) {
    const long slice_bytes = (long)T * kHeadDim * 2;
    auto tile_ok = [&](long row0, const char* what) {
        for (int w = 0; w < kWaves; ++w)
            for (int i = 0; i < 2; ++i)
                for (int l = 0; l < 64; ++l) {
                    const long voff = dlb_global_byte(w, i, l);
                    long off;
                    if (row0 + 64 <= T) {
                        off = row0 * 128 + voff;
                    } else {
                        long r = row0 + (voff >> 7);
                        if (r > T - 1) r = T - 1;
                        off = r * 128 + (voff & 127);
                    }
                    CHECK(off >= 0 && off + 16 <= slice_bytes, "%s tile load outside slice", what);
                }
    };
    const int nkb = (T + kBwdBlockKV - 1) / kBwdBlockKV;
    const int nqt = (T + kBwdBlockQ - 1) / kBwdBlockQ;
    for (int b = 0; b < nkb * BH; ++b) {
        int bh, kb;
        bwd_kv_tile_of(b, nkb * BH, nkb, causal, &bh, &kb);
        CHECK(bh >= 0 && bh < BH, "bwd slice");
        // the single-kernel backward's K block: two 64-row tiles
        tile_ok((long)kb * kBwdBlockKV, "bwd_kvq K block");
        tile_ok((long)kb * kBwdBlockKV + 64, "bwd_kvq K block");
        for (int u = bwd_first_qtile(kb, causal); u < nqt; ++u) {
            const long q0 = (long)u * kBwdBlockQ;
            tile_ok(q0, "bwd_kv");
            for (int l = 0; l < 64; ++l) {
                long r = q0 + l;
                if (r > T - 1) r = T - 1;
                CHECK(r >= 0 && r * 4 + 4 <= (long)T * 4, "lse/delta load");
            }
        }
    }
    const int nq = (T + kBlockM - 1) / kBlockM;
    for (int b = 0; b < nq * BH; ++b) {
        int bh, qt;
        tile_of(b, nq * BH, nq, causal, &bh, &qt);
        const int n = key_tiles(qt, T, kBlockN16, causal);
        for (int u = 0; u < n; ++u) tile_ok((long)u * kBlockN16, "bwd_q");
    }
}

// The decode kernels: every workgroup's key range, each wave's tile loads
// (rows clamped below the range end, inside the slice), the LDS ring and the
// merge area, and the partial-result indices.
template <int D>
static void check_decode(int BH, int Tq, int Tk, bool causal) {
    using G = HeadDim<D>;
    constexpr int kTile = dec_tile_bytes<D>();
    constexpr long kRow = G::kRowBytes;
    int nsplit, chunk;
    decode_plan(BH, Tq, Tk, &nsplit, &chunk);
    CHECK(nsplit >= 1 && chunk % (kWaves * kDecTile) == 0, "decode plan");
    CHECK((long)nsplit * chunk >= Tk && (long)(nsplit - 1) * chunk < Tk, "decode split cover");
    const int nqt = (Tq + kDecTile - 1) / kDecTile;
    const long parts = (long)BH * Tq * nsplit;
    const long ring_bytes = (long)kWaves * 2 * 2 * kTile;
    CHECK(ring_bytes <= 160 * 1024, "decode ring exceeds the LDS");
    CHECK(kTile == 1024 * dec_instr<D>() && 2 * dec_instr<D>() <= 63, "decode tile loads");
    CHECK((long)kWaves * kDecTile * D * 4 + 2 * kWaves * kDecTile * 4 <= ring_bytes,
          "decode merge area exceeds the ring");
    // the merge's threads (query row, D / 8 dims) cover each row once
    {
        std::vector<int> mcov(kDecTile * D, 0);
        for (int tid = 0; tid < kThreads; ++tid)
            for (int j = 0; j < D / 8; ++j) mcov[(tid >> 3) * D + (D / 8) * (tid & 7) + j]++;
        for (int x = 0; x < kDecTile * D; ++x) CHECK(mcov[x] == 1, "decode merge cover");
    }
    // the combine's lanes cover each of a row's D dims once
    {
        const int npl = D >= 64 ? D / 64 : 1;
        std::vector<int> ccov(D, 0);
        for (int lane = 0; lane < 64; ++lane) {
            if (!(D >= 64 || lane < D)) continue;
            const int dim = D >= 64 ? lane : (lane & (D - 1));
            for (int i = 0; i < npl; ++i) {
                CHECK(dim + 64 * i < D, "decode combine dim");
                ccov[dim + 64 * i]++;
            }
        }
        for (int x = 0; x < D; ++x) CHECK(ccov[x] == 1, "decode combine cover");
    }
    std::vector<int> covered((size_t)Tk, 0);
    for (int b = 0; b < BH * nqt * nsplit; ++b) {
        const int per = nqt * nsplit, bh = b / per, rem = b % per;
        const int qt = rem / nsplit, split = rem % nsplit;
        const int last_q = std::min(qt * kDecTile + kDecTile - 1, Tq - 1);
        const int kend_all = causal ? (Tk - Tq + last_q + 1) : Tk;
        const int k_begin = split * chunk;
        const int k_end = std::min(k_begin + chunk, kend_all);
        CHECK(kend_all >= 1 && kend_all <= Tk, "decode key end");
        const int ntile = k_end > k_begin ? (k_end - k_begin + kDecTile - 1) / kDecTile : 0;
        for (int w = 0; w < kWaves; ++w) {
            const int n = ntile > w ? (ntile - w + kWaves - 1) / kWaves : 0;
            for (int t = 0; t < n; ++t) {
                const int k0 = k_begin + kDecTile * (w + kWaves * t);
                CHECK(k0 < k_end, "decode tile past the range");
                if (bh == 0 && qt == nqt - 1)
                    for (int r = 0; r < kDecTile && k0 + r < k_end; ++r) covered[k0 + r]++;
                for (int i = 0; i < dec_instr<D>(); ++i)
                    for (int l = 0; l < 64; ++l)
                        for (int is_v = 0; is_v < 2; ++is_v) {
                            const long voff = G::global_byte(i, l, is_v);
                            CHECK(voff / kRow < kDecTile, "decode load row beyond the tile");
                            long off;
                            if (k0 + kDecTile <= k_end) {
                                off = (long)k0 * kRow + voff;
                            } else {
                                long r = k0 + voff / kRow;
                                if (r > k_end - 1) r = k_end - 1;
                                off = r * kRow + voff % kRow;
                            }
                            CHECK(off >= 0 && off + 16 <= (long)Tk * kRow, "decode load outside slice");
                            CHECK(1024 * i + 16 * l + 16 <= kTile, "decode LDS tile");
                        }
            }
        }
        for (int rq = 0; rq < kDecTile; ++rq) {
            const int qrow = qt * kDecTile + rq;
            if (qrow >= Tq) continue;
            const long p = ((long)bh * Tq + qrow) * nsplit + split;
            CHECK(p >= 0 && p < parts, "decode partial index");
        }
    }
    // the last query tile of a slice sees every key its queries may see, once
    const int kend_last = causal ? Tk : Tk;
    for (int j = 0; j < kend_last; ++j) CHECK(covered[j] == 1, "decode key %d covered %d times", j, covered[j]);
}

// The decode kernels read a 32-key tile of HeadDim<D>'s layout: the K
// fragments (tile nt = 0) and the V^T reads (steps 0, 1) stay in its rows,
// and the direct loads of its D / 16 instructions fill exactly those rows.
template <int D>
static void check_decode_tile() {
    using G = HeadDim<D>;
    constexpr int kTile = dec_tile_bytes<D>();
    for (int is_v = 0; is_v < 2; ++is_v) {
        std::vector<int> cov(kDecTile * G::kChunks, 0);
        for (int i = 0; i < dec_instr<D>(); ++i)
            for (int l = 0; l < 64; ++l) {
                int row, chunk;
                G::src(i, l, is_v, &row, &chunk);
                CHECK(row < kDecTile, "D%d decode load row", D);
                cov[row * G::kChunks + chunk]++;
            }
        for (int x = 0; x < kDecTile * G::kChunks; ++x) CHECK(cov[x] == 1, "D%d decode cover", D);
    }
    for (int l = 0; l < 64; ++l) {
        for (int ks = 0; ks < G::kSteps; ++ks)
            CHECK(G::kfrag(l & 31, l >> 5, 0, ks) + 16 <= kTile, "D%d decode kfrag", D);
        for (int mt = 0; mt < G::kOTiles; ++mt)
            for (int ks = 0; ks < 2; ++ks)
                for (int half = 0; half < 2; ++half)
                    CHECK(G::vtr(l, mt, ks, half) + 8 <= kTile, "D%d decode vtr", D);
    }
}

// HeadDim<64> is the D = 64 kernels' layout byte for byte.
static void check_head_dim64_same() {
    using G = HeadDim<64>;
    for (int r = 0; r < 64; ++r) {
        for (int c = 0; c < 8; ++c) CHECK(G::k_byte(r, c) == k_byte(r, c), "HeadDim<64> k_byte");
        for (int d = 0; d < 64; ++d) CHECK(G::v_byte(r, d) == v_byte(r, d), "HeadDim<64> v_byte");
    }
    for (int l = 0; l < 64; ++l) {
        for (int i = 0; i < 8; ++i)
            for (int is_v = 0; is_v < 2; ++is_v)
                CHECK(G::global_byte(i, l, is_v) == dl_global_byte(i >> 1, i & 1, l, is_v),
                      "HeadDim<64> direct load");
        for (int nt = 0; nt < 2; ++nt)
            for (int ks = 0; ks < 4; ++ks)
                CHECK(G::kfrag(l & 31, l >> 5, nt, ks) == kfrag_byte(l & 31, l >> 5, nt, ks),
                      "HeadDim<64> kfrag");
        for (int mt = 0; mt < 2; ++mt)
            for (int ks = 0; ks < 4; ++ks)
                for (int half = 0; half < 2; ++half)
                    CHECK(G::vtr(l, mt, ks, half) == vtr_byte(l, mt, ks, half), "HeadDim<64> vtr");
        for (int h = 0; h < 2; ++h)
            for (int ks = 0; ks < 4; ++ks) CHECK(G::q_col(h, ks) == q_col16(h, ks), "HeadDim<64> q_col");
    }
    CHECK(dec_tile_bytes<64>() == kDecTileBytes, "decode tile bytes at D = 64");
}

// The pipelined dK/dV kernel masks only the wave's first tile and the last
// tile: every tile strictly between them must need no mask.
static void check_bwd_kv_edges() {
    for (int causal = 0; causal < 2; ++causal)
        for (int T = 1; T <= 1500; T += (T < 300 ? 1 : 37)) {
            const int nkb = (T + kBwdBlockKV - 1) / kBwdBlockKV;
            const int nqt = (T + kBwdBlockQ - 1) / kBwdBlockQ;
            for (int kb = 0; kb < nkb; ++kb) {
                const int n = nqt - bwd_first_qtile(kb, causal);
                CHECK(n >= 1, "bwd kv: block with no query tile");
                for (int w = 0; w < kWaves; ++w) {
                    const int uw = bwd_kv_first_seen(kb, w, n, causal);
                    for (int u = uw + 1; u + 1 < n; ++u)
                        CHECK(!bwd_kv_edge(kb, w, u, T, causal),
                              "bwd kv: middle tile %d of block %d wave %d T %d needs masks", u, kb,
                              w, T);
                    // tiles before uw hold no visible pair for the wave
                    for (int u = 0; u < uw; ++u) {
                        const int q_last = (bwd_first_qtile(kb, causal) + u) * kBwdBlockQ + kBwdBlockQ - 1;
                        CHECK(q_last < kb * kBwdBlockKV + 32 * w, "bwd kv: skipped tile is visible");
                    }
                }
            }
        }
}

// The pipelined dQ kernel masks only the wave's last visible key tile.
static void check_bwd_q_edges() {
    for (int causal = 0; causal < 2; ++causal)
        for (int T = 1; T <= 1500; T += (T < 300 ? 1 : 37)) {
            const int nq = (T + kBlockM - 1) / kBlockM;
            for (int qt = 0; qt < nq; ++qt) {
                const int n = key_tiles(qt, T, kBlockN16, causal);
                for (int w = 0; w < kWaves; ++w) {
                    const int nw = bwd_q_tiles_seen(qt, w, n, causal);
                    const int wq0 = qt * kBlockM + 32 * w;
                    for (int u = 0; u + 1 < nw; ++u)
                        CHECK(!bwd_q_edge(qt, w, u, T, causal),
                              "bwd q: tile %d of query tile %d wave %d T %d needs masks", u, qt,
                              w, T);
                    // tiles past nw hold no key the wave's queries see
                    for (int u = nw; u < n; ++u)
                        CHECK(causal && u * kBlockN16 > wq0 + 31, "bwd q: skipped tile is visible");
                    // every visible key tile is among the first nw
                    if (wq0 < T) CHECK(nw >= 1, "bwd q: a wave with rows sees no tile");
                }
            }
        }
}

// The single-kernel backward (dQ by atomics): the dS^T writes cover the two
// LDS tiles once with the right (key, query); the dQ product's two
// transposed reads pair the same key in every reduction slot and cover the
// block's 128 keys; the four waves' output blocks cover the 64 x 64 tile
// once; and every atomic's row stays inside the slice.
static void check_bwd_atomic_layout() {
    std::vector<int> cov(128 * 64, 0);
    for (int w = 0; w < kWaves; ++w)
        for (int l = 0; l < 64; ++l)
            for (int mt = 0; mt < 2; ++mt)
                for (int g = 0; g < 4; ++g) {
                    const int ql = l & 31, h = l >> 5;
                    const int b = bwd_ds_byte(w, ql, h, mt, g);
                    CHECK(b % 8 == 0 && b >= 0 && b + 8 <= 2 * kTileBytes16, "dS^T write range");
                    for (int e = 0; e < 4; ++e) {
                        const int tile = b / kTileBytes16;
                        int row, dim;
                        decode_b(b % kTileBytes16 + 2 * e, &row, &dim);
                        const int key = 64 * tile + row;
                        // packed value e of group g is accumulator register
                        // 4g + e: query 32mt + acc_row(4g + e, h)
                        CHECK(key == 32 * w + ql, "dS^T write key");
                        CHECK(dim == 32 * mt + acc_row(4 * g + e, h), "dS^T write query");
                        cov[key * 64 + dim]++;
                    }
                }
    for (int x = 0; x < 128 * 64; ++x) CHECK(cov[x] == 1, "dS^T element written %d times", cov[x]);
    // reduction slots: both operands come from btr of a 64-row tile (ks >> 2)
    // at step ks & 3 with the same lane pattern; the row (key) each slot holds
    std::vector<int> keys(128, 0);
    for (int ks = 0; ks < 8; ++ks)
        for (int h = 0; h < 2; ++h)
            for (int s = 0; s < 8; ++s) {
                const int key = 64 * (ks >> 2) + 16 * (ks & 3) + 8 * (s / 4) + 4 * h + s % 4;
                keys[key]++;
            }
    for (int x = 0; x < 128; ++x) CHECK(keys[x] == 1, "dQ product key %d summed %d times", x, keys[x]);
    std::vector<int> out(64 * 64, 0);
    for (int w = 0; w < kWaves; ++w)
        for (int l = 0; l < 64; ++l)
            for (int r = 0; r < 16; ++r) {
                const int qi = 32 * bwd_dq_qhalf(w) + acc_row(r, l >> 5);
                const int d = 32 * bwd_dq_dhalf(w) + (l & 31);
                CHECK(qi >= 0 && qi < 64 && d >= 0 && d < 64, "dQ block range");
                if (qi >= 0 && qi < 64 && d >= 0 && d < 64) out[qi * 64 + d]++;
            }
    for (int x = 0; x < 64 * 64; ++x) CHECK(out[x] == 1, "dQ element owned %d times", out[x]);
}
static void check_bwd_atomic_rows(int T, bool causal) {
    const int nkb = (T + kBwdBlockKV - 1) / kBwdBlockKV;
    const int nqt = (T + kBwdBlockQ - 1) / kBwdBlockQ;
    for (int kb = 0; kb < nkb; ++kb)
        for (int u = 0; u < nqt - bwd_first_qtile(kb, causal); ++u)
            for (int w = 0; w < kWaves; ++w) {
                const int qb = (bwd_first_qtile(kb, causal) + u) * kBwdBlockQ + 32 * bwd_dq_qhalf(w);
                for (int h = 0; h < 2; ++h)
                    for (int r = 0; r < 16; ++r) {
                        const int row = std::min(qb + acc_row(r, h), T - 1);
                        CHECK(row >= 0 && row < T, "dQ atomic row %d outside T %d", row, T);
                    }
            }
}
// The wait at the top of tile u lets 16 operations stay pending; with
// vector-memory operations completing in issue order this covers tile u's
// loads when at least 16 operations were issued after them. Model each wave's
// issue order (K block and tile 0 drained before the loop; loads of tile
// u + 1 at the top of tile u; 16 atomics at its end) and check it.
static void check_bwd_atomic_waits() {
    for (int n = 1; n <= 40; ++n)
        for (int w = 0; w < kWaves; ++w) {
            const int L = 4 + (w < 2 ? 1 : 0);
            std::vector<int> tile_of_op;  // -1: atomic, else the tile loaded
            for (int u = 0; u < n; ++u) {
                if (u > 0) {
                    // ops issued after the last load of tile u
                    int last = -1;
                    for (int i = 0; i < (int)tile_of_op.size(); ++i)
                        if (tile_of_op[i] == u) last = i;
                    CHECK(last >= 0, "tile %d loads never issued", u);
                    const int after = (int)tile_of_op.size() - 1 - last;
                    CHECK(after >= 16, "wait at tile %d of %d: only %d ops after its loads", u, n, after);
                }
                if (u + 1 < n)
                    for (int i = 0; i < L; ++i) tile_of_op.push_back(u + 1);
                for (int i = 0; i < 16; ++i) tile_of_op.push_back(-1);
            }
        }
}

// The fp32 key-split kernel: a wave's 4 x 256-thread staging covers its K
// tile (32 keys x 64 dims) and V^T tile once, inside its LDS slot; the
// waves' tiles (w, w + 8, ...) cover each key tile once, masked tiles being
// exactly those from main_tiles on; the merge area's rows stay inside the
// tiles' LDS.
static void check_fwd32_split() {
    std::vector<int> kc(32 * 64, 0), vc(32 * 64, 0);
    for (int lane = 0; lane < 64; ++lane)
        for (int j = 0; j < 4; ++j) {
            const int t = lane + 64 * j;
            for (int i = 0; i < 2; ++i) {
                int row, col;
                k_stage32(t, i, &row, &col);
                CHECK(row >= 0 && row < 32 && col >= 0 && col + 4 <= 64, "split K stage");
                CHECK(k_lds32(row, col) + 4 <= kKTile32, "split K slot");
                for (int e = 0; e < 4; ++e) kc[row * 64 + col + e]++;
            }
            int key0, dim0;
            v_stage32(t, &key0, &dim0);
            CHECK(key0 >= 0 && key0 + 2 <= 32 && dim0 >= 0 && dim0 + 4 <= 64, "split V stage");
            for (int d = 0; d < 4; ++d) {
                CHECK(v_lds32(dim0 + d, key0) + 2 <= kVTile32, "split V slot");
                for (int e = 0; e < 2; ++e) vc[(key0 + e) * 64 + dim0 + d]++;
            }
        }
    for (int x = 0; x < 32 * 64; ++x) CHECK(kc[x] == 1 && vc[x] == 1, "split staging coverage");
    CHECK(kSplitWaves * kSplitRows * kMergeStride32 + 2 * kSplitWaves * kSplitRows <=
              kSplitWaves * kSplitTileFloats, "split merge area");
    for (int causal = 0; causal < 2; ++causal)
        for (int T = 1; T <= 700; T += (T < 200 ? 1 : 29)) {
            const int nq = (T + kSplitRows - 1) / kSplitRows;
            for (int qt = 0; qt < nq; ++qt) {
                const int n = key_tiles(qt, T, kBlockN32, causal, kSplitRows);
                const int nm = main_tiles(qt, T, kBlockN32, causal, kSplitRows);
                std::vector<int> seen(n, 0);
                for (int w = 0; w < kSplitWaves; ++w)
                    for (int kt = w; kt < n; kt += kSplitWaves) seen[kt]++;
                for (int kt = 0; kt < n; ++kt) CHECK(seen[kt] == 1, "split tile %d owned %d times", kt, seen[kt]);
                // a tile before main_tiles needs no mask for any of the 32 rows
                for (int kt = 0; kt < nm; ++kt)
                    CHECK(kt * 32 + 31 < T && (!causal || kt * 32 + 31 <= qt * kSplitRows),
                          "split main tile %d of qt %d T %d needs a mask", kt, qt, T);
                // every key some row of the tile sees lies in the first n tiles
                const int last_row = std::min(T - 1, qt * kSplitRows + kSplitRows - 1);
                const int last_key = causal ? last_row : T - 1;
                CHECK(last_key < n * 32, "split tiles miss key %d", last_key);
            }
        }
    for (int BH : {1, 3, 6, 48, 64})
        for (int T : {1, 256, 1000, 1024, 4096, 8192})
            CHECK(fwd32_split(BH, T) == (((T + 127) / 128) * BH < 256), "split selection");
}

// Other head dims: direct-load coverage, K fragment decode, strides and bank
// conflicts, and the transposed V reads simulated with the hardware rule
// against the P fragment's key order, for D = 32 and 128.
template <int D>
static void check_head_dim() {
    using G = HeadDim<D>;
    for (int is_v = 0; is_v < 2; ++is_v) {
        std::vector<int> cov(64 * G::kChunks, 0);
        for (int i = 0; i < G::kInstr; ++i)
            for (int l = 0; l < 64; ++l) {
                int row, chunk;
                G::src(i, l, is_v, &row, &chunk);
                CHECK(row >= 0 && row < 64 && chunk >= 0 && chunk < G::kChunks, "D%d src range", D);
                const int want = is_v ? G::v_byte(row, 8 * chunk) : G::k_byte(row, chunk);
                CHECK(1024 * i + 16 * l == want, "D%d direct load slot", D);
                CHECK(G::global_byte(i, l, is_v) == row * G::kRowBytes + chunk * 16, "D%d src", D);
                cov[row * G::kChunks + chunk]++;
            }
        for (int x = 0; x < 64 * G::kChunks; ++x) CHECK(cov[x] == 1, "D%d chunk cover %d", D, cov[x]);
    }
    for (int nt = 0; nt < 2; ++nt)
        for (int ks = 0; ks < G::kSteps; ++ks) {
            for (int l = 0; l < 64; ++l) {
                const int ql = l & 31, h = l >> 5;
                const int b = G::kfrag(ql, h, nt, ks);
                CHECK(b % 16 == 0 && b + 16 <= G::kTileBytes, "D%d kfrag range", D);
                CHECK(b == G::kfrag(ql, h, 0, ks) + 32 * G::kRowBytes * nt, "D%d kfrag stride", D);
                const int row = b / G::kRowBytes, slot = (b % G::kRowBytes) / 16;
                CHECK(row == 32 * nt + ql && (slot ^ G::swz_k(row)) == 2 * ks + h, "D%d kfrag decode", D);
            }
            for (int grp = 0; grp < 4; ++grp) {
                std::vector<int> used(64, 0);
                for (int l = 16 * grp; l < 16 * grp + 16; ++l) {
                    const int b = G::kfrag(l & 31, l >> 5, nt, ks);
                    for (int x = 0; x < 4; ++x) used[(b / 4 + x) % 64]++;
                }
                for (int x = 0; x < 64; ++x) CHECK(used[x] <= 1, "D%d K read bank conflict", D);
            }
        }
    for (int mt = 0; mt < G::kOTiles; ++mt)
        for (int ks = 0; ks < 4; ++ks)
            for (int half = 0; half < 2; ++half) {
                int addr[64];
                for (int l = 0; l < 64; ++l) {
                    addr[l] = G::vtr(l, mt, ks, half);
                    CHECK(addr[l] % 8 == 0 && addr[l] + 8 <= G::kTileBytes, "D%d vtr range", D);
                    CHECK(addr[l] == G::vtr(l, mt, 0, 0) + 16 * G::kRowBytes * ks +
                                         8 * G::kRowBytes * half,
                          "D%d vtr stride", D);
                }
                for (int l = 0; l < 64; ++l) {
                    const int g0 = l & ~15, i = l & 15, h = l >> 5;
                    for (int r = 0; r < 4; ++r) {
                        const int src = g0 + 4 * r + i / 4;
                        const int byte = addr[src] + 2 * (i % 4);
                        const int row = byte / G::kRowBytes;
                        const int slot = (byte % G::kRowBytes) / 16;
                        const int dim = (slot ^ G::swz_v(row)) * 8 + (byte % 16) / 2;
                        const int s8 = 4 * half + r;
                        const int nt = ks >> 1, reg = (ks & 1) * 8 + s8;
                        const int pkey = 32 * nt + acc_row(reg, h);
                        CHECK(row == pkey && dim == 32 * mt + (l & 31),
                              "D%d V tr lane %d slot %d: row %d dim %d", D, l, s8, row, dim);
                    }
                }
                for (int half32 = 0; half32 < 2; ++half32) {
                    std::vector<int> used(64, 0);
                    for (int l = 32 * half32; l < 32 * half32 + 32; ++l)
                        for (int x = 0; x < 2; ++x) used[(addr[l] / 4 + x) % 64]++;
                    for (int x = 0; x < 64; ++x) CHECK(used[x] <= 1, "D%d V tr bank conflict", D);
                }
            }
    for (int h = 0; h < 2; ++h)
        for (int ks = 0; ks < G::kSteps; ++ks)
            CHECK(G::q_col(h, ks) + 8 <= D && G::q_col(h, ks) == 16 * ks + 8 * h, "D%d q_col", D);
}

// The skewed loop of the other head dims (K in two stages, V in three, each
// wave waiting only for K(t) at iteration t): simulate one wave's loads in
// issue order (a wait that leaves w loads in flight completes all older
// ones) and check that every K(t) read (iteration t) and V(t) read
// (iteration t + 1, or after the loop; earlier when the wave has no key
// left to see from tile `skip` on) finds its tile landed in its stage, and
// that no stage is reloaded while a read of its old tile is still to come.
static void check_hd_skew_ring(int n, int skip, int ni) {
    struct Load { int tile; bool v; };
    std::vector<Load> q;
    int done = 0;
    std::vector<int> kst(2, -1), vst(3, -1);
    std::vector<int> kdone(n, 0), vdone(n, 0);
    std::vector<int> vread_at(n, -1);  // iteration whose step reads V(t)
    for (int t = 0; t < n; ++t) {
        if (t < skip) vread_at[t] = t + 1;  // in iteration t+1 (or the end, n)
        else vread_at[t] = -1;              // never computed
    }
    auto issue = [&](int t, int it) {
        // K(t) replaces K(t-2): read in iteration t-2 < it
        const int ko = kst[t % 2];
        if (ko >= 0) CHECK(ko < it, "hd skew: K stage of %d reloaded at %d", ko, it);
        const int vo = vst[t % 3];
        if (vo >= 0 && vread_at[vo] >= 0)
            CHECK(vread_at[vo] < it, "hd skew: V stage of %d reloaded at %d", vo, it);
        kst[t % 2] = t; vst[t % 3] = t;
        for (int i = 0; i < ni; ++i) q.push_back({t, false});
        for (int i = 0; i < ni; ++i) q.push_back({t, true});
    };
    auto wait = [&](int left) {
        while ((int)q.size() - done > left) {
            const Load& l = q[done++];
            if (l.v) vdone[l.tile]++; else kdone[l.tile]++;
        }
    };
    issue(0, -1);
    for (int t = 0; t < n; ++t) {
        wait(ni);
        if (t + 1 < n) issue(t + 1, t);
        if (t >= skip) {
            // flush of V(t-1) if it was computed, then nothing
            if (t == skip && t >= 1) {
                CHECK(vdone[t - 1] == ni && vst[(t - 1) % 3] == t - 1, "hd skew: flushed V(%d)", t - 1);
            }
            continue;
        }
        CHECK(kdone[t] == ni && kst[t % 2] == t, "hd skew: K(%d) at %d", t, t);
        if (t >= 1) CHECK(vdone[t - 1] == ni && vst[(t - 1) % 3] == t - 1, "hd skew: V(%d) at %d", t - 1, t);
    }
    wait(0);
    if (skip >= n && n >= 1)
        CHECK(vdone[n - 1] == ni && vst[(n - 1) % 3] == n - 1, "hd skew: last V(%d)", n - 1);
}

// The K / V rings of the 16-bit kernel: simulate one wave's issue order and
// vmcnt waits (a wait leaving w loads in flight completes all older loads),
// and check that each read finds its tile landed in its stage and that no
// stage is reloaded after the barrier of an iteration that still reads it.
static void check_ring(int n, int n_main) {
    std::vector<int> kst(kRingK, -1), vst(kRingV, -1);  // tile held per stage
    std::vector<int> kdone(n, 0), vdone(n, 0);
    std::vector<int> kread(n, -100), vread(n, -100);     // iteration of last read
    struct Load { int tile; bool v; };
    std::vector<Load> q;  // this wave's loads in issue order
    int done = 0;         // loads completed (a prefix of q)
    auto issue = [&](int u, int it) {
        const int tk = batch_k(u, n), tv = batch_v(u, n);
        if (tk >= 0) {
            const int old = kst[tk % kRingK];
            if (old >= 0) CHECK(kread[old] < it, "K stage of tile %d reloaded at %d", old, it);
            kst[tk % kRingK] = tk;
            q.push_back({tk, false}); q.push_back({tk, false});
        }
        if (tv >= 0) {
            const int old = vst[tv % kRingV];
            if (old >= 0) CHECK(vread[old] < it, "V stage of tile %d reloaded at %d", old, it);
            vst[tv % kRingV] = tv;
            q.push_back({tv, true}); q.push_back({tv, true});
        }
    };
    auto wait = [&](int in_flight) {
        CHECK(in_flight >= 0 && in_flight <= (int)q.size(), "wait count");
        done = (int)q.size() - in_flight;
        for (int i = 0; i < done; ++i) (q[i].v ? vdone : kdone)[q[i].tile] = 1;
    };
    auto needK = [&](int t, int it) {
        CHECK(t >= 0 && t < n && kst[t % kRingK] == t && kdone[t], "K(%d) not ready at %d", t, it);
        kread[t] = it;
    };
    auto needV = [&](int t, int it) {
        CHECK(t >= 0 && t < n && vst[t % kRingV] == t && vdone[t], "V(%d) not ready at %d", t, it);
        vread[t] = it;
    };
    for (int u = -3; u < 0; ++u) issue(u, -1);
    if (n_main > 0) {
        wait(batch_size(-2, n) + batch_size(-1, n));  // K(0)
        needK(0, -1);
        for (int j = 0; j < n_main; ++j) {
            wait(batch_size(j - 1, n));
            issue(j, j);  // after the barrier
            if (j + 1 < n_main) needK(j + 1, j);
            if (j >= 1) needV(j - 1, j);
            needK(j, j);  // the rescale case recomputes S(j)
        }
    }
    // barrier epochs: main iteration j is epoch j; the last product of the
    // main tiles waits for everything, passes a barrier (epoch n_main) and
    // leaves the first edge tile ready; each later edge tile waits and passes
    // a barrier of its own
    int epoch = n_main - 1;
    bool synced = false;
    if (n_main > 0) {
        wait(0);
        ++epoch;
        synced = true;
        needV(n_main - 1, epoch);
    }
    for (int t = n_main; t < n; ++t) {
        if (!synced) {
            wait(0);
            ++epoch;
        }
        synced = false;
        // the edge loop issues nothing: its batches are empty
        CHECK(batch_k(t, n) < 0, "edge iteration %d would load K", t);
        CHECK(batch_v(t, n) < 0, "edge iteration %d would load V", t);
        needK(t, epoch);
        needV(t, epoch);
    }
}

// The eight-wave 16-bit forward: workgroup -> (slice, 256-row query tile)
// is a bijection; each wave computes exactly the key tiles that hold a key
// one of its valid rows sees (w8_seen), the tiles before the first wave's
// masked one need no mask for any wave that computes them, at most four
// tiles follow them (the per-wave masked tail), and the load schedule's
// waits and stage reuse hold for every tile count.
static void check_w8(int BH, int T, bool causal) {
    const int nq = (T + kBlockM8 - 1) / kBlockM8;
    const int total = nq * BH;
    std::vector<int> hit(total, 0);
    for (int b = 0; b < total; ++b) {
        int bh, qt;
        tile_of8(b, total, nq, causal, &bh, &qt);
        CHECK(bh >= 0 && bh < BH && qt >= 0 && qt < nq, "w8 tile_of8(%d)", b);
        if ((total & 7) == 0 && (BH & 7) == 0)  // each XCD keeps whole slices
            CHECK(bh / (BH / 8) == (b & 7), "w8 tile_of8(%d): slice %d off its XCD", b, bh);
        if (bh >= 0 && bh < BH && qt >= 0 && qt < nq) hit[bh * nq + qt]++;
    }
    for (int i = 0; i < total; ++i) CHECK(hit[i] == 1, "w8 tile %d hit %d times", i, hit[i]);
    for (int qt = 0; qt < nq; ++qt) {
        const int n_tiles = key_tiles(qt, T, kBlockN16, causal, kBlockM8);
        const int n_all_main = w8_main(qt, 0, T, causal);
        CHECK(n_all_main >= 0 && n_all_main <= n_tiles && n_tiles - n_all_main <= 4,
              "w8 T %d qt %d: %d unmasked of %d tiles", T, qt, n_all_main, n_tiles);
        CHECK(n_tiles >= 1 && (long)(n_tiles - 1) * kBlockN16 < T, "w8 T %d qt %d: tiles", T, qt);
        for (int w = 0; w < kWaves8; ++w) {
            const int wq0 = qt * kBlockM8 + 32 * w;
            const int rlast = std::min(wq0 + 31, T - 1);
            const int seen = w8_seen(qt, w, T, causal);
            CHECK(seen >= 0 && seen <= n_tiles, "w8 T %d qt %d w %d: seen %d of %d", T, qt, w, seen,
                  n_tiles);
            const int wm = w8_main(qt, w, T, causal);
            CHECK(wm >= 0 && wm <= seen, "w8 main %d > seen %d", wm, seen);
            for (int t = 0; t < n_tiles; ++t) {
                bool vis = false, needs_mask = false;
                for (int r = wq0; r <= rlast; ++r)
                    for (int key = t * kBlockN16; key < (t + 1) * kBlockN16; ++key) {
                        const bool ok = key < T && (!causal || key <= r);
                        vis = vis || ok;
                        needs_mask = needs_mask || !ok;
                    }
                CHECK(vis == (t < seen), "w8 T %d qt %d w %d tile %d: visible %d, seen %d", T, qt,
                      w, t, (int)vis, seen);
                if (t < n_all_main && t < seen)
                    CHECK(!needs_mask, "w8 T %d qt %d w %d: unmasked tile %d needs a mask", T, qt,
                          w, t);
                if (t < wm) CHECK(!needs_mask, "w8 per-wave main tile %d needs a mask", t);
            }
        }
        // ring: tile t in stage t % kRing8, t + kAhead8 issued after the
        // barrier of iteration t; the wait leaves the later issued tiles
        // (2 loads each) pending and needs tile t's loads done
        for (int t = 0; t < n_tiles; ++t) {
            const int issued_before = std::min(t + kAhead8 - 1, n_tiles - 1);  // last tile issued
            const int ahead = std::min(kAhead8 - 1, n_tiles - 1 - t);
            CHECK(ahead == issued_before - t && ahead >= 0 && ahead <= 2, "w8 ring wait at %d", t);
            if (t + kAhead8 < n_tiles)
                CHECK((t + kAhead8) % kRing8 == (t + kRing8 - 1) % kRing8 &&
                          (t + kAhead8) % kRing8 != t % kRing8,
                      "w8 ring stage reuse at %d", t);
        }
    }
    // wave w's direct load is the 4-wave schedule's instruction w: it lands
    // at byte 1024 w of the stage, and the 8 waves cover each tile once
    for (int is_v = 0; is_v < 2; ++is_v) {
        std::vector<int> cov(512, 0);
        for (int w = 0; w < kWaves8; ++w)
            for (int l = 0; l < 64; ++l) {
                int row, chunk;
                dl_src(w >> 1, w & 1, l, is_v, &row, &chunk);
                CHECK(row == 8 * w + l / 8, "w8 direct load row");
                cov[row * 8 + chunk]++;
            }
        for (int i = 0; i < 512; ++i) CHECK(cov[i] == 1, "w8 direct load coverage %d", i);
    }
}

// The key-split form of the eight-wave kernel: workgroup -> (slice, 128-row
// query tile) is a bijection; waves w and w + 4 own the same 32 rows, and in
// iteration i group g computes tile 2i + g when one of those rows sees a key
// in it. Every visible tile is computed by exactly one group, nothing else
// is, the unmasked loop's tiles need no mask, every computed tile was
// issued (the pair of iteration i in the prologue or after iteration
// i - 1's barrier) into a stage no other tile of iterations i - 1 .. i holds,
// and the merge buffers fit in the rings.
static void check_w8_split(int BH, int T, bool causal) {
    constexpr int BM = kBlockM8s, RW = kWaves8 / kSplit8;
    static_assert(kSplit8 == 2 && BM == 32 * RW, "two key groups of four waves");
    static_assert(RW * 32 * 64 * 4 <= kRing8 * kTileBytes16, "O hand-over fits the K ring");
    static_assert(RW * 2 * 64 * 4 <= kRing8 * kTileBytes16, "mc, l hand-over fits the V ring");
    const int nq = (T + BM - 1) / BM;
    const int total = nq * BH;
    std::vector<int> hit(total, 0);
    for (int b = 0; b < total; ++b) {
        int bh, qt;
        tile_of8(b, total, nq, causal, &bh, &qt);
        CHECK(bh >= 0 && bh < BH && qt >= 0 && qt < nq, "w8s tile_of8(%d)", b);
        if (bh >= 0 && bh < BH && qt >= 0 && qt < nq) hit[bh * nq + qt]++;
    }
    for (int i = 0; i < total; ++i) CHECK(hit[i] == 1, "w8s tile %d hit %d times", i, hit[i]);
    for (int qt = 0; qt < nq; ++qt) {
        const int n_tiles = key_tiles(qt, T, kBlockN16, causal, BM);
        const int n_all_main = w8_main(qt, 0, T, causal, BM);
        const int n_iter = (n_tiles + kSplit8 - 1) / kSplit8;
        CHECK(n_tiles >= 1 && n_all_main >= 0 && n_all_main <= n_tiles, "w8s T %d qt %d", T, qt);
        // issue iteration of each tile: the prologue (-1) issues the first
        // pair, iteration i the pair of iteration i + 1
        std::vector<int> issued(n_tiles, -2);
        for (int t = 0; t < kSplit8 && t < n_tiles; ++t) issued[t] = -1;
        for (int i = 0; i < n_iter; ++i)
            for (int j = 0; j < kSplit8; ++j) {
                const int t = kSplit8 * (i + 1) + j;
                if (t < n_tiles) issued[t] = i;
            }
        for (int t = 0; t < n_tiles; ++t) {
            CHECK(issued[t] == t / kSplit8 - 1, "w8s tile %d issued at %d", t, issued[t]);
            // no tile of iterations t/2 - 1 .. t/2 shares its stage
            for (int u = std::max(0, (t / kSplit8 - 1) * kSplit8); u < t; ++u)
                CHECK(u % kRing8 != t % kRing8, "w8s stage of tile %d held by tile %d", t, u);
        }
        for (int rw = 0; rw < RW; ++rw) {
            const int wq0 = qt * BM + 32 * rw;
            const int rlast = std::min(wq0 + 31, T - 1);
            const int seen = w8_seen(qt, rw, T, causal, BM);
            std::vector<int> done(n_tiles, 0);
            for (int g = 0; g < kSplit8; ++g)
                for (int i = 0; i < n_iter; ++i) {
                    const int t = kSplit8 * i + g;
                    if (t >= seen) continue;
                    CHECK(t < n_tiles, "w8s T %d qt %d rw %d: tile %d not loaded", T, qt, rw, t);
                    if (t >= n_tiles) continue;
                    done[t]++;
                    bool needs_mask = false;
                    for (int r = wq0; r <= rlast; ++r)
                        for (int key = t * kBlockN16; key < (t + 1) * kBlockN16; ++key)
                            needs_mask = needs_mask || !(key < T && (!causal || key <= r));
                    if (i < n_all_main / kSplit8)
                        CHECK(!needs_mask, "w8s T %d qt %d rw %d: unmasked tile %d needs a mask",
                              T, qt, rw, t);
                }
            for (int t = 0; t < n_tiles; ++t) {
                bool vis = false;
                for (int r = wq0; r <= rlast; ++r)
                    for (int key = t * kBlockN16; key < (t + 1) * kBlockN16; ++key)
                        vis = vis || (key < T && (!causal || key <= r));
                CHECK(done[t] == (vis ? 1 : 0), "w8s T %d qt %d rw %d tile %d: computed %d times",
                      T, qt, rw, t, done[t]);
            }
        }
    }
}

// Which 16-bit D = 64 forward a call runs: the eight-wave kernel, its key
// split or the 128-row kernel, exactly one; causal calls never take the
// 128-row kernel, and the split's grid (128-row workgroups) is at most twice
// the eight-wave one's.
static void check_fwd16_dispatch() {
    for (long long BH = 1; BH <= 600; BH += (BH < 64 ? 1 : 7))
        for (int T : {1, 64, 200, 256, 257, 1000, 1024, 2048, 4096, 8192, 16384, 32768})
            for (int causal = 0; causal < 2; ++causal) {
                const bool w8 = fwd16_eight_waves(BH, T, causal);
                const bool split = fwd16_key_split(BH, T, causal);
                CHECK(!(w8 && split), "dispatch BH %lld T %d: both", BH, T);
                if (causal) CHECK(w8 || split, "dispatch BH %lld T %d: causal 128-row", BH, T);
                const long long nq8 = (T + kBlockM8 - 1) / kBlockM8;
                if (!causal) CHECK(w8 == (nq8 * BH >= kW8MinGrid), "dispatch full BH %lld T %d", BH, T);
            }
    CHECK(fwd16_eight_waves(48, 8192, true), "the metric workload runs the eight-wave kernel");
    CHECK(fwd16_key_split(48, 1024, true), "4 x 12 x 1024 causal runs the key split");
}

int main() {
    check_direct16();
    check_bwd_layout();
    check_bwd_kv_edges();
    check_bwd_q_edges();
    check_bwd_atomic_layout();
    check_fwd32_split();
    check_bwd_atomic_waits();
    for (int T = 1; T <= 700; T += (T < 300 ? 1 : 23))
        for (int causal = 0; causal < 2; ++causal) check_bwd_atomic_rows(T, causal);
    check_head_dim<32>();
    check_head_dim<64>();
    check_head_dim<128>();
    check_head_dim64_same();
    // the backward's two row arrays: the second starts past the first's last
    // row, on a 256-byte boundary, with under 256 bytes of padding
    for (long long rows = 1; rows <= 70000; rows += (rows < 300 ? 1 : 997)) {
        const long long st = bwd_ws_stride(rows);
        CHECK(st >= rows && st % 64 == 0 && st - rows < 64, "bwd_ws_stride(%lld)", rows);
    }
    CHECK(bwd_ws_stride(4LL * 12 * 8192) == 4LL * 12 * 8192, "bwd_ws_stride of the metric shape");
    for (int n = 1; n <= 40; ++n)
        for (int skip = 0; skip <= n; ++skip)
            for (int ni : {1, 2, 4}) check_hd_skew_ring(n, skip, ni);
    check_decode_tile<32>();
    check_decode_tile<64>();
    check_decode_tile<128>();
    for (int Tk : {1, 2, 31, 32, 33, 127, 128, 129, 300, 1000, 4096, 8192})
        for (int Tq : {1, 2, 7, 31, 32, 33, 64, 100})
            for (int BH : {1, 6, 48})
                for (int causal = 0; causal < 2; ++causal)
                    if (Tq <= Tk) {
                        check_decode<32>(BH, Tq, Tk, causal);
                        check_decode<64>(BH, Tq, Tk, causal);
                        check_decode<128>(BH, Tq, Tk, causal);
                    }
    for (int T : {1, 63, 64, 65, 127, 128, 129, 300, 1000, 8192})
        for (int BH : {1, 6, 48})
            for (int causal = 0; causal < 2; ++causal) {
                check_bwd_map(BH, T, causal);
                check_bwd_access(BH, T, causal);
            }
    for (int T : {1, 2, 63, 64, 65, 127, 128, 129, 200, 255, 256, 300, 1000, 1024, 4096, 8192})
        for (int causal = 0; causal < 2; ++causal) {
            const int nq = (T + kBlockM - 1) / kBlockM;
            for (int qt = 0; qt < nq; ++qt)
                check_ring(key_tiles(qt, T, kBlockN16, causal), main_tiles(qt, T, kBlockN16, causal));
        }
    const int Ts[] = {1, 2, 31, 32, 33, 63, 64, 65, 100, 127, 128, 129, 255, 256,
                      257, 300, 1000, 1024, 4096};
    const int BHs[] = {1, 3, 6, 8, 48};
    for (int T : Ts)
        for (int BH : BHs)
            for (int causal = 0; causal < 2; ++causal) {
                check_tile_map(BH, T, causal);
                check_key_cover(T, kBlockN16, causal);
                check_key_cover(T, kBlockN32, causal);
                check16(BH, T, causal);
                check32(BH, T, causal);
            }
    // the large shapes: tile map and key cover only (enumeration is costly)
    const int bigT[] = {8192, 32768, 131072};
    for (int T : bigT)
        for (int causal = 0; causal < 2; ++causal) {
            check_tile_map(48, T, causal);
            check_tile_map(16, T, causal);
            check_key_cover(T, kBlockN16, causal);
            check_key_cover(T, kBlockN32, causal);
        }
    check16(48, 8192, true);
    for (int T : {1, 2, 31, 32, 33, 63, 64, 65, 100, 127, 128, 129, 200, 255, 256, 257, 300, 511,
                  512, 513, 700, 1000, 1024, 1100, 2048, 4096})
        for (int BH : {1, 3, 8, 48})
            for (int causal = 0; causal < 2; ++causal) check_w8(BH, T, causal);
    for (int causal = 0; causal < 2; ++causal) check_w8(1, 8192, causal);
    for (int T : {1, 2, 63, 64, 65, 127, 128, 129, 191, 192, 193, 255, 256, 257, 300, 513, 1000,
                  1024, 2100, 4096})
        for (int BH : {1, 3, 8, 16})
            for (int causal = 0; causal < 2; ++causal) check_w8_split(BH, T, causal);
    check_fwd16_dispatch();
    if (failures) {
        std::printf("%d failures\n", failures);
        return 1;
    }
    std::printf("layout ok\n");
    return 0;
}
