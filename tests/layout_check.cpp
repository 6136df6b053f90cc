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
    }
}

static void check16(int BH, int T, bool causal) {
    const long tensor = (long)BH * T * kHeadDim;
    const int nq = (T + kBlockM - 1) / kBlockM;
    // LDS stage coverage (independent of the tile index)
    std::vector<int> kcov(kKTile16, 0), vcov(kVTile16, 0);
    for (int t = 0; t < kThreads; ++t) {
        for (int i = 0; i < 2; ++i) {
            int row, col;
            k_stage16(t, i, &row, &col);
            const int a = k_lds16(row, col);
            CHECK(row >= 0 && row < kBlockN16 && col >= 0 && col + 8 <= kHeadDim, "k_stage16");
            CHECK(a % 8 == 0 && a + 8 <= kKTile16, "k_lds16 %d", a);
            for (int x = 0; x < 8; ++x) kcov[a + x]++;
        }
        int key0, dim0;
        v_stage16(t, &key0, &dim0);
        CHECK(key0 % 2 == 0 && key0 + 2 <= kBlockN16 && dim0 + 8 <= kHeadDim, "v_stage16");
        for (int j = 0; j < 8; ++j) {
            const int a = v_lds16(dim0 + j, key0);
            CHECK(a % 2 == 0 && a + 2 <= kVTile16, "v_lds16 %d", a);
            CHECK(v_lds16(dim0 + j, key0 + 1) == a + 1, "key pair not adjacent");
            vcov[a]++;
            vcov[a + 1]++;
        }
    }
    for (int r = 0; r < kBlockN16; ++r)
        for (int c = 0; c < kHeadDim; ++c)
            CHECK(kcov[k_lds16(r, c)] == 1, "K lds (%d,%d) written %d times", r, c,
                  kcov[k_lds16(r, c)]);
    for (int d = 0; d < kHeadDim; ++d)
        for (int key = 0; key < kBlockN16; ++key)
            CHECK(vcov[v_lds16(d, key)] == 1, "V lds (%d,%d) written %d times", d, key,
                  vcov[v_lds16(d, key)]);
    // fragment reads, and the pairing of reduction indices
    for (int lane = 0; lane < 64; ++lane) {
        const int ql = lane & 31, hh = lane >> 5;
        for (int ks = 0; ks < 4; ++ks) {
            const int qc = q_col16(hh, ks);
            CHECK(qc % 8 == 0 && qc + 8 <= kHeadDim, "q_col16");
            for (int nt = 0; nt < 2; ++nt) {
                const int a = kfrag16(ql, hh, nt, ks);
                CHECK(a % 8 == 0 && a + 8 <= kKTile16, "kfrag16");
                // A slot s of K = K[32nt + ql][qc + s]; B slot s of Q = dim qc + s
                CHECK(a == k_lds16(32 * nt + ql, qc), "K/Q dim pairing");
            }
            for (int mt = 0; mt < 2; ++mt) {
                const int a = vfrag16(ql, hh, mt, ks);
                CHECK(a % 8 == 0 && a + 8 <= kVTile16, "vfrag16");
                for (int s = 0; s < 8; ++s) {
                    // key of P slot s of step ks (accumulator register r0 + s)
                    const int nt = ks >> 1, r = (ks & 1) * 8 + s;
                    const int pkey = 32 * nt + acc_row(r, hh);
                    // key of V^T slot s at row 32mt + ql
                    CHECK(a + s == v_lds16(32 * mt + ql, pkey),
                          "P/V key mismatch lane %d ks %d slot %d", lane, ks, s);
                }
            }
        }
        for (int mt = 0; mt < 2; ++mt)
            for (int g = 0; g < 4; ++g) {
                const int d = 32 * mt + acc_row(4 * g, hh);
                CHECK(d % 4 == 0 && d + 4 <= kHeadDim, "O store dims");
            }
    }
    // global accesses of every workgroup
    const int total = nq * BH;
    for (int b = 0; b < total; ++b) {
        int bh, qt;
        tile_of(b, total, nq, causal, &bh, &qt);
        const long base = (long)bh * T * kHeadDim;
        const int n = key_tiles(qt, T, kBlockN16, causal);
        for (int kt = 0; kt < n; ++kt) {
            const int k0 = kt * kBlockN16;
            for (int t = 0; t < kThreads; ++t) {
                for (int i = 0; i < 2; ++i) {
                    int row, col;
                    k_stage16(t, i, &row, &col);
                    if (k0 + row < T) {
                        const long a = base + (long)(k0 + row) * kHeadDim + col;
                        CHECK(a >= 0 && a + 8 <= tensor && a % 8 == 0, "K global");
                    }
                }
                int key0, dim0;
                v_stage16(t, &key0, &dim0);
                for (int e = 0; e < 2; ++e)
                    if (k0 + key0 + e < T) {
                        const long a = base + (long)(k0 + key0 + e) * kHeadDim + dim0;
                        CHECK(a >= 0 && a + 8 <= tensor && a % 8 == 0, "V global");
                    }
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

int main() {
    // vt_pos16 is a permutation of one 64-key tile that keeps pairs adjacent
    std::set<int> pos;
    for (int key = 0; key < kBlockN16; ++key) pos.insert(vt_pos16(key));
    CHECK((int)pos.size() == kBlockN16 && *pos.begin() == 0 &&
              *pos.rbegin() == kBlockN16 - 1, "vt_pos16 not a permutation");
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
    if (failures) {
        std::printf("%d failures\n", failures);
        return 1;
    }
    std::printf("layout ok\n");
    return 0;
}
