// Host-side internals shared by the C-ABI entry points (mgemm_api.cpp) and
// the measured dispatch table (dispatch.cpp).
#pragma once

#include <hip/hip_runtime.h>

#include <map>
#include <tuple>

#include "../../include/mgemm.h"
#include "common.h"

namespace mgemm_host {

using mgemm::Problem;

// A kernel and its number of K ranges (1: no split).
struct Choice {
    mgemm_kernel_t k;
    int ksplit;
};

// Table key of a canonical problem: dtype, operand layouts and either the
// exact shape (bucket == 0) or ceil(log2) of each size (bucket == 1).
using TableKey = std::tuple<int, int, int, int, int64_t, int64_t, int64_t>;

// A table entry: a kernel and the split requested from it (0 = the
// library's choice), normalised per problem when used.
struct TableEntry {
    int kernel;
    int ksplit;
    double us;
};

struct Table {
    std::map<TableKey, TableEntry> entries;
};

TableKey exact_key(const Problem& p);
TableKey bucket_key(const Problem& p);
int ceil_log2(int64_t x);

}  // namespace mgemm_host

struct mgemm_handle_s {
    int device;
    int num_cu;
    mgemm::Workspace ws;          // device memory owned by the handle
    mgemm_host::Table table;      // measured choices (mgemm_tune / mgemm_table_import)
    unsigned long long* stamps;   // clock-stamp buffer (mgemm_set_clock_stamps), or null
    int64_t stamps_cap;           // workgroups it has room for
};

namespace mgemm_host {

mgemm_status_t make_problem(mgemm_handle_t h, mgemm_layout_t layoutA, mgemm_layout_t layoutB,
                            int64_t M, int64_t N, int64_t K, float alpha, const void* A,
                            int64_t lda, const void* B, int64_t ldb, float beta, void* C,
                            int64_t ldc, mgemm_dtype_t dtype, Problem* out);
bool variant_supports(const Problem& p, mgemm_kernel_t k);
// Number of K ranges a forced kernel runs with for a request (0 = its own
// choice); 0 when it cannot run them.
int forced_splits(const Problem& p, const mgemm::Workspace& ws, mgemm_kernel_t k, int requested);
// The built-in time model's choice.
Choice model_choice(const Problem& p, const mgemm::Workspace& ws);
// Table entry, else the model.
Choice choose(mgemm_handle_t h, const Problem& p);
Choice choose_in(const Table* table, const mgemm::Workspace& ws, const Problem& p);
mgemm_status_t launch(mgemm_handle_t h, const Problem& p, Choice c, hipStream_t s);
mgemm_status_t launch_ws(const mgemm::Workspace& ws, const Problem& p, Choice c, hipStream_t s);
bool splittable(mgemm_kernel_t k);
mgemm_status_t make_problem_on(int num_cu, mgemm_layout_t layoutA, mgemm_layout_t layoutB,
                               int64_t M, int64_t N, int64_t K, float alpha, const void* A,
                               int64_t lda, const void* B, int64_t ldb, float beta, void* C,
                               int64_t ldc, mgemm_dtype_t dtype, Problem* out);
// The body of mgemm_run_variant for a device with num_cu compute units, a
// workspace and an optional dispatch table.  A forced variant whose split
// (or stream-K) form needs more workspace than ws holds returns too_big.
mgemm_status_t run_core(int num_cu, const mgemm::Workspace& ws, const Table* table,
                        mgemm_kernel_t forced, int ksplit, mgemm_layout_t layoutA,
                        mgemm_layout_t layoutB, int64_t M, int64_t N, int64_t K, float alpha,
                        const void* A, int64_t lda, const void* B, int64_t ldb, float beta,
                        void* C, int64_t ldc, mgemm_dtype_t dtype, mgemm_epilogue_t epilogue,
                        hipStream_t stream, mgemm_status_t too_big,
                        unsigned long long* stamps = nullptr, int64_t stamps_cap = 0);

}  // namespace mgemm_host
