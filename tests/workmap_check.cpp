// Host-side check of the forward's workgroup map (kernel_common.h): for
// many shapes, with and without folded row blocks and with split keys, every
// workgroup of the grid is mapped with map_item and every query slot with
// item_row / slot_head, exactly as the kernels do. Checks that every
// (batch, query head, row < Sq, key range) is held by exactly one slot, that
// a workgroup's heads share its KV head, that rows stay below the
// workgroup's row_end, and that each wave's first and last slots hold its
// smallest and largest row (the kernels' idle-wave test and causal stop
// rely on both). Built with hipcc (the header includes the HIP runtime) and
// run by tests/test_workmap.py.
#include <cstdio>
#include <cstdint>
#include <vector>

#include "kernel_common.h"

static long bad = 0, maps = 0;

static void fail(const char* what, int B, int Hq, int Hkv, int Sq, int fold, int ns, int pid) {
    if (bad < 10)
        std::printf("FAIL %s: B=%d Hq=%d Hkv=%d Sq=%d fold=%d n_split=%d pid=%d\n", what, B, Hq, Hkv, Sq, fold, ns, pid);
    ++bad;
}

static void check_map(attn::FwdParams p, bool causal) {
    attn::set_divisors(p);
    ++maps;
    const int B = p.B, Hq = p.Hq, Hkv = p.Hkv, Sq = p.Sq, ns = p.n_split;
    const int grid = p.n_units * p.n_row_blocks * ns;
    std::vector<uint8_t> seen((size_t)B * Hq * Sq * ns, 0);
    const int slots = 4 * 32;   // four query waves of 32 slots (two row blocks of 64 when folded)
    for (int pid = 0; pid < grid; ++pid) {
        const attn::WorkItem w = attn::map_item(p, causal, pid);
        if (w.b < 0 || w.b >= B || w.hkv < 0 || w.hkv >= Hkv || w.split < 0 || w.split >= ns) {
            fail("item out of range", B, Hq, Hkv, Sq, p.fold, ns, pid);
            continue;
        }
        for (int wave = 0; wave * 32 < slots; ++wave) {
            int lo = 1 << 30, hi = -1;
            for (int n = 0; n < 32; ++n) {
                const int s = 32 * wave + n;
                const int row = attn::item_row(p, w, s);
                const int hq = w.hq0 + attn::slot_head(p, s);
                lo = row < lo ? row : lo;
                hi = row > hi ? row : hi;
                if (hq / (Hq / Hkv) != w.hkv) fail("head outside the KV head's group", B, Hq, Hkv, Sq, p.fold, ns, pid);
                if (row < 0) fail("negative row", B, Hq, Hkv, Sq, p.fold, ns, pid);
                if (row >= Sq) continue;
                if (row >= w.row_end) fail("row past row_end", B, Hq, Hkv, Sq, p.fold, ns, pid);
                uint8_t& c = seen[(((size_t)w.b * Hq + hq) * Sq + row) * ns + w.split];
                if (c) fail("slot held twice", B, Hq, Hkv, Sq, p.fold, ns, pid);
                c = 1;
            }
            if (attn::item_row(p, w, 32 * wave) != lo || attn::item_row(p, w, 32 * wave + 31) != hi)
                fail("wave's first / last slot not its smallest / largest row", B, Hq, Hkv, Sq, p.fold, ns, pid);
        }
    }
    for (size_t i = 0; i < seen.size(); ++i)
        if (!seen[i]) {
            fail("row never mapped", B, Hq, Hkv, Sq, p.fold, ns, -1);
            break;
        }
}

int main() {
    const int shapes[][4] = {   // B, Hq, Hkv, Sq
        {1, 32, 1, 1024}, {1, 32, 32, 1024}, {1, 4, 4, 545}, {1, 8, 2, 600}, {1, 2, 2, 650},
        {2, 32, 8, 4096}, {4, 16, 16, 2048}, {1, 8, 1, 1000}, {3, 15, 5, 130}, {3, 32, 8, 200},
        {5, 6, 3, 70}, {8, 32, 8, 1}, {32, 32, 1, 4}, {2, 16, 4, 2}, {1, 4, 2, 10}, {2, 8, 2, 5},
        {1, 64, 8, 1024}, {3, 6, 3, 999}, {1, 2, 1, 33}, {2, 12, 4, 257}, {1, 1, 1, 1}, {1, 16, 16, 4096},
        {8, 32, 1, 1024}, {1, 3, 3, 700}, {2, 2, 2, 64},
    };
    for (const auto& sh : shapes)
        for (int causal = 0; causal < 2; ++causal)
            for (int ns : {1, 3}) {
                attn::FwdParams p{};
                p.B = sh[0]; p.Hq = sh[1]; p.Hkv = sh[2]; p.Sq = sh[3]; p.Skv = sh[3];
                p.G = p.Hq / p.Hkv;
                p.n_split = ns;
                attn::set_slot_map(p, true, 32, 4, true);
                check_map(p, causal);
                if (attn::fold_row_blocks(p)) check_map(p, causal);
            }
    std::printf("maps %ld, failures %ld\n", maps, bad);
    return bad != 0;
}
