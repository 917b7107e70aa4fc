// Optional checks of the device inputs of the compute calls, on when the
// environment holds SPECVERIFY_VALIDATE=1 (read at every call).
//
// Without them the kernels clamp out-of-range indices and the results for
// such inputs are unspecified (the header's conventions).  With them each
// call first waits for its stream, copies the index and logit inputs to host
// memory and checks the preconditions the header states: page ids of every
// page a call touches in [0, num_blocks), lengths within the declared
// capacity, tokens in [0, V), uniforms in [0, 1), finite temperatures and
// top-p values, logits without NaN or +inf and with a finite entry per row.
// The first violation is printed to stderr (call, array, index, value) and
// returned as SV_ERR_BAD_INPUT before anything is launched.  After the
// launches the call waits for the stream again, so a device error is
// reported by the call that caused it (SV_ERR_HIP).  Host memory only; a
// debugging aid, slow by design.
#ifndef SV_VALIDATE_H_
#define SV_VALIDATE_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

bool validate_on();

// Pages of sequence b over positions [0, kv_len[b] + extra): ids in
// [0, num_blocks), 0 <= kv_len[b] <= max_len (max_len < 0: no bound), and
// kv_len[b] + extra <= 16 * max_blocks_per_seq.
int check_pages(const char* fn, const int32_t* block_table, const int32_t* kv_len, int B,
                int extra, int num_blocks, int max_blocks_per_seq, int max_len, hipStream_t st);

// The commit's slots: L0 = kv_len[b] - n - 1 >= 0 with n = num_accepted[b]
// in [0, N), pages of [0, L0 + N) in range; nodes[b][j] in [0, N) when given.
int check_commit(const char* fn, const int32_t* block_table, const int32_t* kv_len,
                 const int32_t* num_accepted, const int32_t* nodes, int B, int N, int num_blocks,
                 int max_blocks_per_seq, hipStream_t st);

// Logit rows [rows, V] of dtype: no NaN or +inf, at least one finite entry.
int check_logits(const char* fn, const char* name, const void* x, long long rows, int V,
                 int dtype, hipStream_t st);

// Integers in [0, V); entries with (i % stride) < skip are not checked.
int check_tokens(const char* fn, const int32_t* tok, long long n, int V, int stride, int skip,
                 hipStream_t st);

// Parent lists [B, N] of trees in topological order: parents[b][0] = -1,
// 0 <= parents[b][i] < i.
int check_parents(const char* fn, const int32_t* parents, int B, int N, hipStream_t st);

// Floats: unit = true, in [0, 1) (uniforms); false, finite (temperature,
// top_p).
int check_floats(const char* fn, const char* name, const float* x, long long n, bool unit,
                 hipStream_t st);

// After the launches: wait for the stream, map a device error to SV_ERR_HIP.
int finish(const char* fn, hipStream_t st, int status);

}  // namespace sv

#endif  // SV_VALIDATE_H_
