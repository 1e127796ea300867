// Host-only driver for the planner, built with the address and
// undefined-behaviour sanitizers by tests/test_plan_sanitized.py (g++, no GPU
// code).  It feeds seeded random rank tables -- valid ones and ones the planner
// must reject -- to sketchssm_plan_create / _export / _destroy, exports into
// arrays of exactly the documented sizes (so any write past them is caught)
// and checks the tables' invariants: frames sorted by (group, rank) and
// distinct, offsets are running sums, buckets follow the rank, and the order is
// a permutation with dense heads first and buckets non-increasing.
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

#include "sketchssm.h"

static int fail(const char* what, int iter) {
    std::fprintf(stderr, "invariant broken at iteration %d: %s\n", iter, what);
    return 1;
}

int main(int argc, char** argv) {
    const int iters = argc > 1 ? std::atoi(argv[1]) : 2000;
    std::mt19937 rng(12345);
    int accepted = 0, rejected = 0;
    for (int it = 0; it < iters; ++it) {
        sketchssm_shape sh{};
        sh.B = 1 + int(rng() % 64);
        sh.H = 1 + int(rng() % 256);
        sh.K = 128;
        sh.V = (int[]){64, 80, 128}[rng() % 3];
        sh.W = 16;
        sh.G = 1 + int(rng() % 8);
        sh.basis_rows = 1 + int(rng() % 79);
        sh.rank_cap = 1 + int(rng() % 64);
        sh.kind = SKSSM_MAMBA2 + int(rng() % 3);
        sh.qkv = int(rng() % 2);
        const int rmax = std::min(std::min(sh.rank_cap, sh.basis_rows), sh.K);
        const bool bad = rng() % 5 == 0;
        std::vector<int32_t> rank(sh.H), group(sh.H);
        for (int h = 0; h < sh.H; ++h) {
            rank[h] = rng() % 4 == 0 ? 0 : 1 + int(rng() % rmax);
            group[h] = int(rng() % sh.G);
        }
        if (bad) {
            const int h = int(rng() % sh.H);
            if (rng() % 2) rank[h] = rmax + 1 + int(rng() % 8);
            else group[h] = sh.G + int(rng() % 3);
        }
        sketchssm_plan* plan = nullptr;
        const sketchssm_status st = sketchssm_plan_create(&sh, rank.data(), group.data(), &plan);
        if (bad) {
            if (st != SKSSM_ESHAPE || plan) return fail("bad table accepted", it);
            ++rejected;
            continue;
        }
        if (st != SKSSM_OK || !plan) return fail("valid table rejected", it);
        ++accepted;
        int32_t F = -1;
        if (sketchssm_plan_export(plan, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                  nullptr, &F) != SKSSM_OK || F < 0)
            return fail("frame count", it);
        std::vector<int32_t> fi(sh.H), fro(F + 1), zro(sh.H + 1), bucket(sh.H), order(sh.H),
            fg(F > 0 ? F : 1), fr(F > 0 ? F : 1);
        if (sketchssm_plan_export(plan, fi.data(), fro.data(), zro.data(), bucket.data(),
                                  order.data(), fg.data(), fr.data(), &F) != SKSSM_OK)
            return fail("export", it);
        for (int f = 0; f < F; ++f) {
            if (fr[f] < 1 || fr[f] > rmax) return fail("frame rank", it);
            if (fro[f + 1] != fro[f] + fr[f]) return fail("frame row offsets", it);
            if (f > 0 && !(fg[f - 1] < fg[f] || (fg[f - 1] == fg[f] && fr[f - 1] < fr[f])))
                return fail("frames not sorted and distinct", it);
        }
        if (fro[0] != 0 || zro[0] != 0) return fail("offsets start", it);
        std::vector<int> seen(sh.H, 0);
        for (int h = 0; h < sh.H; ++h) {
            if (zro[h + 1] != zro[h] + rank[h]) return fail("z row offsets", it);
            const int want = rank[h] == 0 ? 0 : 1 + (rank[h] - 1) / 8;
            if (bucket[h] != want) return fail("bucket", it);
            if (rank[h] == 0 ? fi[h] != -1
                             : (fi[h] < 0 || fi[h] >= F || fg[fi[h]] != group[h] || fr[fi[h]] != rank[h]))
                return fail("frame index", it);
            if (order[h] < 0 || order[h] >= sh.H || seen[order[h]]++) return fail("order permutation", it);
        }
        for (int p = 1; p < sh.H; ++p) {
            const int a = bucket[order[p - 1]], b = bucket[order[p]];
            const bool ok = (a == 0) ? true : (b != 0 && (a > b || (a == b && order[p - 1] < order[p])));
            if (!ok) return fail("launch order", it);
        }
        const size_t ze = sketchssm_z_elems(plan), fe = sketchssm_frame_elems(plan);
        if (ze != size_t(sh.B) * sh.V * zro[sh.H] || fe != size_t(sh.K) * fro[F])
            return fail("element counts", it);
        sketchssm_plan_destroy(plan);
    }
    std::printf("ok accepted=%d rejected=%d\n", accepted, rejected);
    return 0;
}
