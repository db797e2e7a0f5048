// Measured dispatch table: the tuner (mgemm_tune), the table's text form
// (mgemm_table_export / mgemm_table_import) and the call-weighted choice.
//
// "Chapter 5: Operators and Runtime" (ai-infra-book), section 5.4.5: rule out
// the implementations that cannot run, time the rest on representative
// shapes, keep the cheapest; its Example 5-9: one implementation serving
// several shapes is judged by the total time over the calls, each shape
// weighted by how often it is called.  Section 5.5.3: similar shapes share a
// choice through buckets.  Here every kernel handles any shape, so a bucket
// shares the choice only (no padding); the buckets are powers of two in M, N
// and K of the canonical problem.
#include <hip/hip_runtime.h>

#include <cmath>
#include <algorithm>
#include <map>
#include <string>
#include <vector>

#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "host.h"

namespace mgemm_host {

int ceil_log2(int64_t x) {
    int l = 0;
    while (l < 62 && ((int64_t)1 << l) < x) ++l;
    return l;
}

TableKey exact_key(const Problem& p) {
    return TableKey{0, p.dtype, p.a_kc, p.b_kc, p.M, p.N, p.K};
}

TableKey bucket_key(const Problem& p) {
    return TableKey{1, p.dtype, p.a_kc, p.b_kc, ceil_log2(p.M), ceil_log2(p.N), ceil_log2(p.K)};
}

namespace {

const char* dtype_name(int d) { return d == mgemm::F32 ? "f32" : d == mgemm::F16 ? "f16" : "bf16"; }

int dtype_of(const char* s) {
    if (!strcmp(s, "f32")) return mgemm::F32;
    if (!strcmp(s, "f16")) return mgemm::F16;
    if (!strcmp(s, "bf16")) return mgemm::BF16;
    return -1;
}

int kernel_of(const char* s) {
    for (int k = 1; k < MGEMM_KERNEL_COUNT; ++k)
        if (!strcmp(s, mgemm_kernel_name((mgemm_kernel_t)k))) return k;
    return -1;
}

// Mean time of one call of variant c (microseconds): two warm-up calls, one
// call to size the runs, then the best of two runs of 3..50 calls (about
// 2 ms each).  Consecutive calls use the operand sets in turn (probs[i % n]),
// so memory-bound shapes are timed streaming from HBM rather than from the
// 256 MiB last-level cache.  +inf if a launch fails.
double time_choice(mgemm_handle_t h, const std::vector<Problem>& probs, Choice c, hipStream_t s,
                   hipEvent_t e0, hipEvent_t e1) {
    const size_t np = probs.size();
    size_t next = 0;
    auto run = [&]() { return launch(h, probs[next++ % np], c, s) == MGEMM_SUCCESS; };
    for (int i = 0; i < 2; ++i)
        if (!run()) return INFINITY;
    float ms = 0.f;
    if (hipEventRecord(e0, s) != hipSuccess || !run() ||
        hipEventRecord(e1, s) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
        hipEventElapsedTime(&ms, e0, e1) != hipSuccess)
        return INFINITY;
    int reps = (int)(2.0 / (ms > 1e-4f ? ms : 1e-4f));
    reps = reps < 3 ? 3 : (reps > 50 ? 50 : reps);
    double best = INFINITY;
    for (int round = 0; round < 2; ++round) {
        if (hipEventRecord(e0, s) != hipSuccess) return INFINITY;
        for (int i = 0; i < reps; ++i)
            if (!run()) return INFINITY;
        if (hipEventRecord(e1, s) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
            hipEventElapsedTime(&ms, e0, e1) != hipSuccess)
            return INFINITY;
        const double us = 1e3 * ms / reps;
        if (us < best) best = us;
    }
    return best;
}

// Splits requested from split-capable kernels while tuning.
const int TUNE_SPLITS[] = {1, 2, 3, 4, 5, 6, 8, 10, 12, 16, 24, 32};

struct DeviceBuffers {
    void* a = nullptr;    // `sets` consecutive copies of the largest A
    void* b = nullptr;    // and of the largest B
    void* c = nullptr;
    ~DeviceBuffers() {
        if (a) (void)hipFree(a);
        if (b) (void)hipFree(b);
        if (c) (void)hipFree(c);
    }
};

// Operand sets for the timing runs: enough copies that the largest A and B
// together exceed twice the 256 MiB last-level cache, at most 64.
int operand_sets(size_t ab_bytes) {
    const size_t want = (size_t)512 << 20;
    size_t n = ab_bytes ? (want + ab_bytes - 1) / ab_bytes : 1;
    return (int)(n < 1 ? 1 : (n > 64 ? 64 : n));
}

struct Events {
    hipEvent_t e0 = nullptr, e1 = nullptr;
    ~Events() {
        if (e0) (void)hipEventDestroy(e0);
        if (e1) (void)hipEventDestroy(e1);
    }
};

}  // namespace
}  // namespace mgemm_host

using namespace mgemm_host;

extern "C" {

int32_t mgemm_weighted_choice(int32_t n_shapes, int32_t n_variants, const double* times,
                              const double* calls) {
    if (n_shapes < 1 || n_variants < 1 || times == nullptr) return -1;
    for (int s = 0; s < n_shapes; ++s)
        if (calls && !(calls[s] >= 0.0 && std::isfinite(calls[s]))) return -1;
    int32_t best = -1;
    double best_total = INFINITY;
    for (int v = 0; v < n_variants; ++v) {
        double total = 0.0;
        bool ok = true;
        for (int s = 0; s < n_shapes && ok; ++s) {
            const double w = calls ? calls[s] : 1.0;
            if (w == 0.0) continue;
            const double t = times[(size_t)s * n_variants + v];
            if (!(t >= 0.0 && std::isfinite(t))) ok = false;
            else total += w * t;
        }
        if (ok && total < best_total) {
            best_total = total;
            best = v;
        }
    }
    return best;
}

mgemm_status_t mgemm_tune(mgemm_handle_t h, mgemm_dtype_t dtype, mgemm_layout_t layoutA,
                          mgemm_layout_t layoutB, int32_t n, const int64_t* M, const int64_t* N,
                          const int64_t* K, const double* calls, mgemm_tune_result_t* results,
                          hipStream_t stream) {
    if (!h || n < 1 || !M || !N || !K) return MGEMM_ERR_INVALID_ARG;
    if (dtype != MGEMM_F32 && dtype != MGEMM_F16 && dtype != MGEMM_BF16) return MGEMM_ERR_INVALID_ARG;
    if ((layoutA != MGEMM_ROW_MAJOR && layoutA != MGEMM_COL_MAJOR) ||
        (layoutB != MGEMM_ROW_MAJOR && layoutB != MGEMM_COL_MAJOR))
        return MGEMM_ERR_INVALID_ARG;
    const int64_t lim = (int64_t)1 << 34;          // elements per operand
    int64_t na = 0, nb = 0, nc = 0;
    for (int i = 0; i < n; ++i) {
        if (M[i] < 1 || N[i] < 1 || K[i] < 1 || M[i] > lim || N[i] > lim || K[i] > lim)
            return MGEMM_ERR_INVALID_ARG;
        if (M[i] > lim / K[i] || K[i] > lim / N[i] || M[i] > lim / N[i]) return MGEMM_ERR_INVALID_ARG;
        if (calls && !(calls[i] >= 0.0 && std::isfinite(calls[i]))) return MGEMM_ERR_INVALID_ARG;
        na = M[i] * K[i] > na ? M[i] * K[i] : na;
        nb = K[i] * N[i] > nb ? K[i] * N[i] : nb;
        nc = M[i] * N[i] > nc ? M[i] * N[i] : nc;
    }
    const size_t es = dtype == MGEMM_F32 ? 4 : 2;
    // Round A and B up to 256-byte multiples so every set stays aligned.
    const size_t a_bytes = ((size_t)na * es + 255) & ~(size_t)255;
    const size_t b_bytes = ((size_t)nb * es + 255) & ~(size_t)255;
    const int sets = operand_sets(a_bytes + b_bytes);
    DeviceBuffers buf;
    Events ev;
    if (hipMalloc(&buf.a, a_bytes * sets) != hipSuccess || hipMalloc(&buf.b, b_bytes * sets) != hipSuccess ||
        hipMalloc(&buf.c, (size_t)nc * es) != hipSuccess || hipEventCreate(&ev.e0) != hipSuccess ||
        hipEventCreate(&ev.e1) != hipSuccess)
        return MGEMM_ERR_HIP;
    if (mgemm::launch_fill_pattern(buf.a, (int64_t)(a_bytes * sets / es), (int)dtype, 1u, stream) != hipSuccess ||
        mgemm::launch_fill_pattern(buf.b, (int64_t)(b_bytes * sets / es), (int)dtype, 2u, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
        return MGEMM_ERR_HIP;

    // Candidate variants: every kernel, split-capable ones at each requested split.
    std::vector<Choice> cands;
    for (int k = 1; k < MGEMM_KERNEL_COUNT; ++k) {
        if (splittable((mgemm_kernel_t)k))
            for (int r : TUNE_SPLITS) cands.push_back({(mgemm_kernel_t)k, r});
        else
            cands.push_back({(mgemm_kernel_t)k, 1});
    }
    const int nv = (int)cands.size();
    std::vector<double> times((size_t)n * nv, INFINITY);
    std::vector<Problem> probs(n);
    std::map<TableKey, TableEntry> add;
    const bool rowA = layoutA == MGEMM_ROW_MAJOR, rowB = layoutB == MGEMM_ROW_MAJOR;

    for (int i = 0; i < n; ++i) {
        const int64_t lda = rowA ? K[i] : M[i], ldb = rowB ? N[i] : K[i], ldc = rowA ? N[i] : M[i];
        std::vector<Problem> set_probs(sets);
        for (int r = 0; r < sets; ++r) {
            mgemm_status_t st = make_problem(h, layoutA, layoutB, M[i], N[i], K[i], 1.0f,
                                             (char*)buf.a + a_bytes * r, lda, (char*)buf.b + b_bytes * r,
                                             ldb, 0.0f, buf.c, ldc, dtype, &set_probs[r]);
            if (st != MGEMM_SUCCESS) return st;
        }
        Problem& p = probs[i];
        p = set_probs[0];
        // Each (kernel, ranges actually used) is timed once per shape.
        std::map<std::pair<int, int>, double> seen;
        auto measure = [&](Choice c) {
            auto key = std::make_pair((int)c.k, c.ksplit);
            auto it = seen.find(key);
            if (it != seen.end()) return it->second;
            const double t = time_choice(h, set_probs, c, stream, ev.e0, ev.e1);
            seen[key] = t;
            return t;
        };
        bool any = false;
        std::vector<std::pair<int, int>> vkey(nv, std::make_pair(-1, 0));
        for (int pass = 0; pass < 2 && !any; ++pass) {
            // The scalar kernel only when nothing else runs the shape.
            for (int v = 0; v < nv; ++v) {
                const mgemm_kernel_t k = cands[v].k;
                if ((k == MGEMM_KERNEL_GENERAL) != (pass == 1) || !variant_supports(p, k)) continue;
                const int ks = forced_splits(p, h->ws, k, cands[v].ksplit);
                if (ks < 1) continue;
                const double t = measure({k, ks});
                vkey[v] = std::make_pair((int)k, ks);
                times[(size_t)i * nv + v] = t;
                any = any || std::isfinite(t);
            }
        }
        if (!any) {
            (void)hipGetLastError();        // clear a failed launch's error
            return MGEMM_ERR_UNSUPPORTED;
        }
        // Close contenders (the three fastest within 15% of the best) are
        // timed twice more, interleaved, and keep their best time, so that one
        // run disturbed by a clock dip does not decide the entry.
        {
            std::vector<std::pair<double, std::pair<int, int>>> order;
            for (const auto& kv : seen)
                if (std::isfinite(kv.second)) order.push_back({kv.second, kv.first});
            std::sort(order.begin(), order.end());
            size_t top = 0;
            while (top < order.size() && top < 3 && order[top].first <= order[0].first * 1.15) ++top;
            if (top > 1)
                for (int round = 0; round < 2; ++round)
                    for (size_t j = 0; j < top; ++j) {
                        const Choice c{(mgemm_kernel_t)order[j].second.first, order[j].second.second};
                        const double t = time_choice(h, set_probs, c, stream, ev.e0, ev.e1);
                        double& kept = seen[order[j].second];
                        if (t < kept) kept = t;
                    }
            for (int v = 0; v < nv; ++v)
                if (vkey[v].first >= 0) times[(size_t)i * nv + v] = seen[vkey[v]];
        }
        int best = 0;
        for (int v = 1; v < nv; ++v)
            if (times[(size_t)i * nv + v] < times[(size_t)i * nv + best]) best = v;
        add[exact_key(p)] = TableEntry{(int)cands[best].k, cands[best].ksplit, times[(size_t)i * nv + best]};
        if (results) {
            const Choice m = model_choice(p, h->ws);
            results[i].chosen = mgemm_variant_t{(int32_t)cands[best].k, cands[best].ksplit};
            results[i].chosen_us = (float)times[(size_t)i * nv + best];
            results[i].model = mgemm_variant_t{(int32_t)m.k, m.ksplit};
            results[i].model_us = (float)measure(m);
        }
    }

    // Buckets: the variant with the smallest call-weighted total over the
    // bucket's shapes (only variants that run all of them).
    std::map<TableKey, std::vector<int>> groups;
    for (int i = 0; i < n; ++i) groups[bucket_key(probs[i])].push_back(i);
    for (const auto& g : groups) {
        const int ns = (int)g.second.size();
        std::vector<double> sub((size_t)ns * nv), w(ns);
        for (int j = 0; j < ns; ++j) {
            const int i = g.second[j];
            w[j] = calls ? calls[i] : 1.0;
            for (int v = 0; v < nv; ++v) sub[(size_t)j * nv + v] = times[(size_t)i * nv + v];
        }
        const int v = mgemm_weighted_choice(ns, nv, sub.data(), w.data());
        if (v < 0) continue;
        double total = 0.0;
        for (int j = 0; j < ns; ++j) total += w[j] * sub[(size_t)j * nv + v];
        add[g.first] = TableEntry{(int)cands[v].k, cands[v].ksplit, total};
    }
    for (const auto& e : add) h->table.entries[e.first] = e.second;
    return MGEMM_SUCCESS;
}

mgemm_status_t mgemm_table_export(mgemm_handle_t h, char* buf, size_t cap, size_t* len) {
    if (!h || !len) return MGEMM_ERR_INVALID_ARG;
    std::string out = "# mgemm dispatch table: exact|bucket dtype a_kc b_kc M|log2M N|log2N K|log2K kernel ksplit us\n";
    char line[256];
    for (const auto& e : h->table.entries) {
        const TableKey& k = e.first;
        snprintf(line, sizeof line, "%s %s %d %d %lld %lld %lld %s %d %.3f\n",
                 std::get<0>(k) ? "bucket" : "exact", dtype_name(std::get<1>(k)), std::get<2>(k),
                 std::get<3>(k), (long long)std::get<4>(k), (long long)std::get<5>(k),
                 (long long)std::get<6>(k), mgemm_kernel_name((mgemm_kernel_t)e.second.kernel),
                 e.second.ksplit, e.second.us);
        out += line;
    }
    *len = out.size();
    if (buf == nullptr && cap == 0) return MGEMM_SUCCESS;
    if (buf == nullptr || cap < out.size() + 1) return MGEMM_ERR_INVALID_ARG;
    memcpy(buf, out.c_str(), out.size() + 1);
    return MGEMM_SUCCESS;
}

mgemm_status_t mgemm_table_import(mgemm_handle_t h, const char* text) {
    if (!h || !text) return MGEMM_ERR_INVALID_ARG;
    std::map<TableKey, TableEntry> add;
    const char* s = text;
    while (*s) {
        const char* e = strchr(s, '\n');
        const size_t n = e ? (size_t)(e - s) : strlen(s);
        std::string line(s, n);
        s += n + (e ? 1 : 0);
        const size_t first = line.find_first_not_of(" \t\r");
        if (first == std::string::npos || line[first] == '#') continue;
        char kind[16], dt[16], kname[64];
        int akc, bkc, ks;
        long long m, nn, k;
        double us;
        char extra;
        if (sscanf(line.c_str(), "%15s %15s %d %d %lld %lld %lld %63s %d %lf %c", kind, dt, &akc,
                   &bkc, &m, &nn, &k, kname, &ks, &us, &extra) != 10)
            return MGEMM_ERR_INVALID_ARG;
        const int bucket = !strcmp(kind, "bucket") ? 1 : (!strcmp(kind, "exact") ? 0 : -1);
        const int d = dtype_of(dt), kern = kernel_of(kname);
        if (bucket < 0 || d < 0 || kern < 0 || (akc != 0 && akc != 1) || (bkc != 0 && bkc != 1) ||
            ks < 0 || ks > MGEMM_MAX_KSPLIT || (ks > 1 && !splittable((mgemm_kernel_t)kern)) ||
            !(us >= 0.0) || m < (bucket ? 0 : 1) || nn < (bucket ? 0 : 1) || k < (bucket ? 0 : 1) ||
            (bucket && (m > 62 || nn > 62 || k > 62)))
            return MGEMM_ERR_INVALID_ARG;
        add[TableKey{bucket, d, akc, bkc, m, nn, k}] = TableEntry{kern, ks, us};
    }
    for (const auto& e : add) h->table.entries[e.first] = e.second;
    return MGEMM_SUCCESS;
}

mgemm_status_t mgemm_table_clear(mgemm_handle_t h) {
    if (!h) return MGEMM_ERR_INVALID_ARG;
    h->table.entries.clear();
    return MGEMM_SUCCESS;
}

}  // extern "C"
