// C ABI of the calibrated block-sparse attention library (declared in
// include/calibatt.h).  Every argument is checked here, on the host, before
// anything is enqueued; the checks make no HIP call, so they also run on a
// machine without a GPU.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/calibatt.h"
#include "launch.h"

namespace {

thread_local std::string g_last_error;

calibatt_status fail(calibatt_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

calibatt_status ok() {
  g_last_error.clear();
  return CALIBATT_OK;
}

calibatt_status hip_fail(hipError_t e, const char* what) {
  return fail(CALIBATT_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

std::mutex g_cu_mutex;
int g_cu_count[64] = {0};

hipError_t cu_count(int* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) {
    *out = 256;
    return hipSuccess;
  }
  std::lock_guard<std::mutex> lk(g_cu_mutex);
  if (g_cu_count[dev] == 0) {
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    g_cu_count[dev] = n > 0 ? n : 1;
  }
  *out = g_cu_count[dev];
  return hipSuccess;
}

// Shape checks common to the attention and pooling entry points.
calibatt_status check_qkv_shape(int B, int H, int L, int seq_len, int d, calibatt_dtype dt,
                                int block) {
  if (dt != CALIBATT_BF16 && dt != CALIBATT_F32) return fail(CALIBATT_ERR_DTYPE, "unknown dtype code %d", (int)dt);
  if (B < 1 || H < 1) return fail(CALIBATT_ERR_SHAPE, "B=%d and H=%d must be >= 1", B, H);
  if (block != 64 && block != 128) return fail(CALIBATT_ERR_UNSUPPORTED, "block=%d (supported: 64, 128)", block);
  if (d != 64 && d != 128) return fail(CALIBATT_ERR_UNSUPPORTED, "d=%d (supported: 64, 128)", d);
  if (L < block || L % block != 0) return fail(CALIBATT_ERR_SHAPE, "L=%d must be a positive multiple of block=%d", L, block);
  if (seq_len < 1 || seq_len > L) return fail(CALIBATT_ERR_SHAPE, "seq_len=%d must be in [1, L=%d]", seq_len, L);
  const long long elems = (long long)B * H * L * d;
  if (elems >= (1LL << 31)) return fail(CALIBATT_ERR_SHAPE, "B*H*L*d=%lld must be < 2^31", elems);
  return CALIBATT_OK;
}

calibatt_status check_ptrs4(const void* Q, const void* K, const void* V, const void* O) {
  if (!Q || !K || !V || !O) return fail(CALIBATT_ERR_NULL, "Q, K, V and O must be non-NULL");
  if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16))
    return fail(CALIBATT_ERR_ALIGN, "Q, K, V and O must be 16-byte aligned");
  return CALIBATT_OK;
}

// Two [B, H, L, d] tensors of `bytes` bytes each share memory.
bool overlap(const void* p, const void* q, uintptr_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
  return a < b + bytes && b < a + bytes;
}

uintptr_t tensor_bytes(int B, int H, int L, int d, calibatt_dtype dt) {
  return (uintptr_t)B * H * L * d * (dt == CALIBATT_F32 ? 4 : 2);
}

// The kernels read V in either layout (natural, or V^T with
// CALIBATT_V_BHDL); no copy of it is made.
calibatt_status check_v_layout(calibatt_vlayout v_layout) {
  if (v_layout != CALIBATT_V_BHLD && v_layout != CALIBATT_V_BHDL)
    return fail(CALIBATT_ERR_SHAPE, "unknown v_layout code %d", (int)v_layout);
  return CALIBATT_OK;
}

// The softmax scale multiplies every score; a non-positive or non-finite one
// has no meaning for the method and would give non-finite outputs.
calibatt_status check_scale(float scale) {
  if (!(scale > 0.f) || !std::isfinite(scale))
    return fail(CALIBATT_ERR_SHAPE, "scale=%g must be finite and > 0", (double)scale);
  return CALIBATT_OK;
}

// O is written while other workgroups still read Q, K and V, so it may not
// share memory with them.
calibatt_status check_out_alias(const void* Q, const void* K, const void* V, const void* O, int B, int H, int L,
                                int d, calibatt_dtype dt) {
  const uintptr_t bytes = tensor_bytes(B, H, L, d, dt);
  if (overlap(O, Q, bytes) || overlap(O, K, bytes) || overlap(O, V, bytes))
    return fail(CALIBATT_ERR_SHAPE, "O must not overlap Q, K or V");
  return CALIBATT_OK;
}

calibatt_status enqueue_transpose(const void* V, void* Vt, int B, int H, int L, int seq_len, int d,
                                  calibatt_dtype dt, void* stream) {
  calibatt::TransposeArgs t;
  t.V = V;
  t.Vt = Vt;
  t.B = B;
  t.H = H;
  t.L = L;
  t.seq_len = seq_len;
  t.d = d;
  t.dtype_f32 = dt == CALIBATT_F32;
  hipError_t e = calibatt::launch_transpose_v(t, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "launching the V transpose");
  return CALIBATT_OK;
}

calibatt_status run_attention(const void* Q, const void* K, const void* V, void* O,
                              const int32_t* row_ptr, const int32_t* col_idx, int block, float scale,
                              int B, int H, int L, int seq_len, int d, calibatt_dtype dt,
                              const int32_t* work_order, int32_t* queue_ws, calibatt_vlayout v_layout,
                              bool dense, void* stream) {
  int ncu = 256;
  if (queue_ws) {
    hipError_t e = cu_count(&ncu);
    if (e != hipSuccess) return hip_fail(e, "querying the compute-unit count");
  }
  calibatt::AttnArgs a;
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.O = O;
  a.row_ptr = row_ptr;
  a.col_idx = col_idx;
  a.work_order = work_order;
  a.queue = queue_ws;
  a.B = B;
  a.H = H;
  a.L = L;
  a.seq_len = seq_len;
  a.d = d;
  a.block = block;
  a.nkb_valid = (seq_len + block - 1) / block;
  a.scale = scale;
  a.dtype_f32 = dt == CALIBATT_F32;
  a.v_transposed = v_layout == CALIBATT_V_BHDL;
  a.num_cu = ncu;
  hipError_t e = calibatt::launch_attention(a, dense, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, dense ? "launching dense attention" : "launching sparse attention");
  return ok();
}

// Checks shared by the sparse entry points: tensors, shape, V layout, scale,
// O aliasing and the kept-block list's pointers and size.
calibatt_status check_sparse_args(const void* Q, const void* K, const void* V, void* O, const int32_t* row_ptr,
                                  const int32_t* col_idx, int block, float scale, int B, int H, int L, int seq_len,
                                  int d, calibatt_dtype dt, const int32_t* work_order, int64_t nnz,
                                  calibatt_vlayout v_layout) {
  calibatt_status s = check_ptrs4(Q, K, V, O);
  if (s != CALIBATT_OK) return s;
  s = check_qkv_shape(B, H, L, seq_len, d, dt, block);
  if (s != CALIBATT_OK) return s;
  s = check_v_layout(v_layout);
  if (s != CALIBATT_OK) return s;
  s = check_scale(scale);
  if (s != CALIBATT_OK) return s;
  s = check_out_alias(Q, K, V, O, B, H, L, d, dt);
  if (s != CALIBATT_OK) return s;
  if (!row_ptr) return fail(CALIBATT_ERR_NULL, "row_ptr must be non-NULL");
  if (nnz < 0) return fail(CALIBATT_ERR_CSR, "nnz=%lld must be >= 0", (long long)nnz);
  const long long rows = (long long)H * (L / block);
  const long long nkb_valid = (seq_len + block - 1) / block;
  if (nnz > rows * nkb_valid)
    return fail(CALIBATT_ERR_CSR, "nnz=%lld exceeds rows*nkb_valid=%lld", (long long)nnz, rows * nkb_valid);
  if (nnz > 0 && !col_idx) return fail(CALIBATT_ERR_NULL, "col_idx must be non-NULL when nnz > 0");
  if (!aligned(row_ptr, 4) || (col_idx && !aligned(col_idx, 4)) || (work_order && !aligned(work_order, 4)))
    return fail(CALIBATT_ERR_ALIGN, "row_ptr, col_idx and work_order must be 4-byte aligned");
  return CALIBATT_OK;
}

}  // namespace

// Scratch of calibatt_sparse_attn_fwd_noalloc: the persistent launch's
// partition counters (kQueueInts int32 = 512 bytes, one 64-byte line per
// partition).  Each GPU the library runs on holds its own copy until the
// process ends.  In host code the name stands for no device address: the
// address used in launches is the one hipGetSymbolAddress returns for the
// current device, kept in g_scratch_ptr.
static __device__ __align__(256) int32_t scratch[calibatt::kQueueInts];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
int32_t* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up on the first
// call there.
calibatt_status scratch_ptr(int32_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "querying the current device");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(CALIBATT_ERR_UNSUPPORTED, "device %d: the static scratch serves devices 0..%d", dev,
                kMaxDevices - 1);
  std::lock_guard<std::mutex> lk(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "looking up the static scratch on the current device");
    if (!p || !aligned(p, 256)) return fail(CALIBATT_ERR_HIP, "the static scratch has no 256-byte aligned address");
    g_scratch_ptr[dev] = static_cast<int32_t*>(p);
  }
  *out = g_scratch_ptr[dev];
  return CALIBATT_OK;
}

}  // namespace

extern "C" {

calibatt_status calibatt_sparse_attn_fwd_noalloc(const void* Q, const void* K, const void* V, void* O,
                                                 const int32_t* row_ptr, const int32_t* col_idx, int block,
                                                 float scale, int B, int H, int L, int seq_len, int d,
                                                 calibatt_dtype dt, const int32_t* work_order, int64_t nnz,
                                                 calibatt_vlayout v_layout, void* stream) {
  calibatt_status s = check_sparse_args(Q, K, V, O, row_ptr, col_idx, block, scale, B, H, L, seq_len, d, dt,
                                        work_order, nnz, v_layout);
  if (s != CALIBATT_OK) return s;
  // The persistent launch needs kQueueInts counters whatever the problem
  // size, so no accepted size outgrows the array.
  int32_t* queue = nullptr;
  s = scratch_ptr(&queue);
  if (s != CALIBATT_OK) return s;
  return run_attention(Q, K, V, O, row_ptr, col_idx, block, scale, B, H, L, seq_len, d, dt, work_order, queue,
                       v_layout, false, stream);
}

calibatt_status calibatt_sparse_attn_fwd(const void* Q, const void* K, const void* V, void* O,
                                         const int32_t* row_ptr, const int32_t* col_idx, int block,
                                         float scale, int B, int H, int L, int seq_len, int d,
                                         calibatt_dtype dt, const int32_t* work_order,
                                         int32_t* queue_ws, int64_t nnz, calibatt_vlayout v_layout,
                                         void* stream) {
  calibatt_status s = check_sparse_args(Q, K, V, O, row_ptr, col_idx, block, scale, B, H, L, seq_len, d, dt,
                                        work_order, nnz, v_layout);
  if (s != CALIBATT_OK) return s;
  if (queue_ws && !aligned(queue_ws, 16)) return fail(CALIBATT_ERR_ALIGN, "queue_ws must be 16-byte aligned");
  return run_attention(Q, K, V, O, row_ptr, col_idx, block, scale, B, H, L, seq_len, d, dt, work_order,
                       queue_ws, v_layout, false, stream);
}

calibatt_status calibatt_dense_attn_fwd(const void* Q, const void* K, const void* V, void* O,
                                        int block, float scale, int B, int H, int L, int seq_len,
                                        int d, calibatt_dtype dt, int32_t* queue_ws,
                                        calibatt_vlayout v_layout, void* stream) {
  calibatt_status s = check_ptrs4(Q, K, V, O);
  if (s != CALIBATT_OK) return s;
  s = check_qkv_shape(B, H, L, seq_len, d, dt, block);
  if (s != CALIBATT_OK) return s;
  s = check_v_layout(v_layout);
  if (s != CALIBATT_OK) return s;
  s = check_scale(scale);
  if (s != CALIBATT_OK) return s;
  s = check_out_alias(Q, K, V, O, B, H, L, d, dt);
  if (s != CALIBATT_OK) return s;
  if (queue_ws && !aligned(queue_ws, 16)) return fail(CALIBATT_ERR_ALIGN, "queue_ws must be 16-byte aligned");
  return run_attention(Q, K, V, O, nullptr, nullptr, block, scale, B, H, L, seq_len, d, dt, nullptr,
                       queue_ws, v_layout, true, stream);
}

calibatt_status calibatt_transpose_v(const void* V, void* Vt, int B, int H, int L, int seq_len, int d,
                                     calibatt_dtype dt, void* stream) {
  if (!V || !Vt) return fail(CALIBATT_ERR_NULL, "V and Vt must be non-NULL");
  if (!aligned(V, 16) || !aligned(Vt, 16)) return fail(CALIBATT_ERR_ALIGN, "V and Vt must be 16-byte aligned");
  calibatt_status s = check_qkv_shape(B, H, L, seq_len, d, dt, 64);
  if (s != CALIBATT_OK) return s;
  if (overlap(V, Vt, tensor_bytes(B, H, L, d, dt)))
    return fail(CALIBATT_ERR_SHAPE, "the transpose is out of place: V and Vt must not overlap");
  s = enqueue_transpose(V, Vt, B, H, L, seq_len, d, dt, stream);
  if (s != CALIBATT_OK) return s;
  return ok();
}

calibatt_status calibatt_block_mass(const void* Q, const void* K, int B, int H, int L, int seq_len,
                                    int d, calibatt_dtype dt, int block, float scale, float* lse_ws,
                                    float* mass, void* stream) {
  if (!Q || !K || !lse_ws || !mass) return fail(CALIBATT_ERR_NULL, "Q, K, lse_ws and mass must be non-NULL");
  if (!aligned(Q, 16) || !aligned(K, 16)) return fail(CALIBATT_ERR_ALIGN, "Q and K must be 16-byte aligned");
  if (!aligned(lse_ws, 4) || !aligned(mass, 4)) return fail(CALIBATT_ERR_ALIGN, "lse_ws and mass must be 4-byte aligned");
  calibatt_status s = check_qkv_shape(B, H, L, seq_len, d, dt, block);
  if (s != CALIBATT_OK) return s;
  s = check_scale(scale);
  if (s != CALIBATT_OK) return s;
  if (dt != CALIBATT_BF16) return fail(CALIBATT_ERR_UNSUPPORTED, "block_mass supports bf16 inputs only");
  if (L / block > calibatt::kMaxKeyBlocks)
    return fail(CALIBATT_ERR_UNSUPPORTED, "L/block=%d exceeds %d key blocks", L / block, calibatt::kMaxKeyBlocks);
  calibatt::MassArgs a;
  a.Q = Q;
  a.K = K;
  a.lse = lse_ws;
  a.mass = mass;
  a.B = B;
  a.H = H;
  a.L = L;
  a.seq_len = seq_len;
  a.d = d;
  a.block = block;
  a.nkb_valid = (seq_len + block - 1) / block;
  a.scale = scale;
  hipError_t e = calibatt::launch_block_mass(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "launching block mass");
  return ok();
}

size_t calibatt_block_mass_ws_bytes(int B, int H, int L, int block) {
  if (B < 1 || H < 1 || (block != 64 && block != 128) || L < block || L % block != 0) return 0;
  return (size_t)B * H * (L / block) * L * sizeof(float);
}

calibatt_status calibatt_block_mass_single_pass(const void* Q, const void* K, int B, int H, int L, int seq_len,
                                                int d, calibatt_dtype dt, int block, float scale, float* lse_ws,
                                                float* mass, void* ws, size_t ws_bytes, void* stream) {
  if (!Q || !K || !lse_ws || !mass || !ws) return fail(CALIBATT_ERR_NULL, "Q, K, lse_ws, mass and ws must be non-NULL");
  if (!aligned(Q, 16) || !aligned(K, 16)) return fail(CALIBATT_ERR_ALIGN, "Q and K must be 16-byte aligned");
  if (!aligned(lse_ws, 4) || !aligned(mass, 4) || !aligned(ws, 256))
    return fail(CALIBATT_ERR_ALIGN, "lse_ws and mass must be 4-byte aligned, ws 256-byte aligned");
  calibatt_status s = check_qkv_shape(B, H, L, seq_len, d, dt, block);
  if (s != CALIBATT_OK) return s;
  s = check_scale(scale);
  if (s != CALIBATT_OK) return s;
  if (dt != CALIBATT_BF16) return fail(CALIBATT_ERR_UNSUPPORTED, "block_mass supports bf16 inputs only");
  if (L / block > calibatt::kMaxKeyBlocks)
    return fail(CALIBATT_ERR_UNSUPPORTED, "L/block=%d exceeds %d key blocks", L / block, calibatt::kMaxKeyBlocks);
  const size_t need = calibatt_block_mass_ws_bytes(B, H, L, block);
  if (ws_bytes < need) return fail(CALIBATT_ERR_CAPACITY, "ws_bytes=%zu, need %zu", ws_bytes, need);
  calibatt::MassArgs a;
  a.Q = Q;
  a.K = K;
  a.lse = lse_ws;
  a.mass = mass;
  a.B = B;
  a.H = H;
  a.L = L;
  a.seq_len = seq_len;
  a.d = d;
  a.block = block;
  a.nkb_valid = (seq_len + block - 1) / block;
  a.scale = scale;
  hipError_t e = calibatt::launch_block_mass_single(a, static_cast<float*>(ws), (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "launching single-pass block mass");
  return ok();
}

size_t calibatt_compile_ws_bytes(int P, int H, int nqb, int nkb) {
  if (P < 1 || H < 1 || nqb < 1 || nkb < 1) return 0;
  const size_t rows = (size_t)H * nqb;
  const size_t keep = (rows * nkb + 15) / 16 * 16;
  return keep + rows * sizeof(int32_t);
}

static calibatt_status compile_common(const float* mass, int P, int H, int nqb, int nkb, int nkb_valid,
                                      int keep_topk, bool energy, long long eps_num, long long eps_den,
                                      int min_agree, int32_t* row_ptr, int32_t* col_idx, int64_t nnz_cap,
                                      int32_t* work_order, int64_t* nnz_out, void* ws, size_t ws_bytes,
                                      void* stream) {
  if (!mass || !row_ptr || !nnz_out || !ws) return fail(CALIBATT_ERR_NULL, "mass, row_ptr, nnz_out and ws must be non-NULL");
  if (P < 1 || H < 1 || nqb < 1 || nkb < 1) return fail(CALIBATT_ERR_SHAPE, "P, H, nqb and nkb must be >= 1");
  if (nkb > calibatt::kMaxKeyBlocks) return fail(CALIBATT_ERR_UNSUPPORTED, "nkb=%d exceeds %d", nkb, calibatt::kMaxKeyBlocks);
  if (nkb_valid < 0 || nkb_valid > nkb) return fail(CALIBATT_ERR_SHAPE, "nkb_valid=%d must be in [0, nkb=%d]", nkb_valid, nkb);
  if (keep_topk < 0) return fail(CALIBATT_ERR_SHAPE, "keep_topk=%d must be >= 0", keep_topk);
  if (min_agree < 0 || min_agree > P) return fail(CALIBATT_ERR_SHAPE, "min_agree=%d must be in [0, P=%d]", min_agree, P);
  if (nnz_cap < 0) return fail(CALIBATT_ERR_SHAPE, "nnz_cap must be >= 0");
  if (nnz_cap > 0 && !col_idx) return fail(CALIBATT_ERR_NULL, "col_idx must be non-NULL when nnz_cap > 0");
  const long long rows = (long long)H * nqb;
  if (rows * nkb >= (1LL << 31)) return fail(CALIBATT_ERR_SHAPE, "H*nqb*nkb must be < 2^31");
  if ((long long)P * rows * nkb >= (1LL << 40)) return fail(CALIBATT_ERR_SHAPE, "P*H*nqb*nkb too large");
  const size_t need = calibatt_compile_ws_bytes(P, H, nqb, nkb);
  if (ws_bytes < need) return fail(CALIBATT_ERR_CAPACITY, "ws_bytes=%zu < %zu required", ws_bytes, need);
  if (!aligned(ws, 16) || !aligned(mass, 4) || !aligned(row_ptr, 4) || (col_idx && !aligned(col_idx, 4)) ||
      (work_order && !aligned(work_order, 4)))
    return fail(CALIBATT_ERR_ALIGN, "ws must be 16-byte aligned; mass, row_ptr, col_idx, work_order 4-byte aligned");
  if (work_order && nqb > calibatt::kMaxKeyBlocks) return fail(CALIBATT_ERR_UNSUPPORTED, "nqb=%d exceeds %d", nqb, calibatt::kMaxKeyBlocks);
  if (work_order && H > calibatt::kMaxHeads) return fail(CALIBATT_ERR_UNSUPPORTED, "H=%d exceeds %d", H, calibatt::kMaxHeads);

  calibatt::CompileArgs a;
  a.mass = mass;
  a.P = P;
  a.H = H;
  a.nqb = nqb;
  a.nkb = nkb;
  a.nkb_valid = nkb_valid;
  a.keep_topk = keep_topk;
  a.min_agree = min_agree;
  a.energy = energy;
  a.eps_num = eps_num;
  a.eps_den = eps_den;
  a.row_ptr = row_ptr;
  a.col_idx = col_idx;
  a.keep_ws = static_cast<uint8_t*>(ws);
  a.count_ws = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(ws) + (rows * nkb + 15) / 16 * 16);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = calibatt::launch_compile_count(a, st);
  if (e != hipSuccess) return hip_fail(e, "launching mask compile (count)");
  int32_t total = 0;
  e = hipMemcpyAsync(&total, row_ptr + rows, sizeof(int32_t), hipMemcpyDeviceToHost, st);
  if (e != hipSuccess) return hip_fail(e, "reading the kept count");
  e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e, "synchronising after mask compile (count)");
  *nnz_out = total;
  if (total > nnz_cap)
    return fail(CALIBATT_ERR_CAPACITY, "kept blocks %d exceed nnz_cap=%lld", total, (long long)nnz_cap);
  if (total > 0) {
    e = calibatt::launch_compile_fill(a, st);
    if (e != hipSuccess) return hip_fail(e, "launching mask compile (fill)");
  }
  if (work_order) {
    e = calibatt::launch_schedule(row_ptr, H, nqb, work_order, st);
    if (e != hipSuccess) return hip_fail(e, "launching work-order build");
  }
  return ok();
}

calibatt_status calibatt_compile_masks(const float* mass, int P, int H, int nqb, int nkb,
                                       int nkb_valid, int keep_topk, int min_agree, int32_t* row_ptr,
                                       int32_t* col_idx, int64_t nnz_cap, int32_t* work_order, int64_t* nnz_out,
                                       void* ws, size_t ws_bytes, void* stream) {
  return compile_common(mass, P, H, nqb, nkb, nkb_valid, keep_topk, false, 0, 1, min_agree, row_ptr, col_idx,
                        nnz_cap, work_order, nnz_out, ws, ws_bytes, stream);
}

calibatt_status calibatt_compile_masks_energy(const float* mass, int P, int H, int nqb, int nkb,
                                              int nkb_valid, int64_t eps_num, int64_t eps_den, int min_agree,
                                              int32_t* row_ptr, int32_t* col_idx, int64_t nnz_cap,
                                              int32_t* work_order, int64_t* nnz_out, void* ws, size_t ws_bytes,
                                              void* stream) {
  if (eps_den < 1 || eps_den > 2147483647LL || eps_num < 0 || eps_num > eps_den)
    return fail(CALIBATT_ERR_SHAPE, "eps = %lld/%lld must satisfy 0 <= eps_num <= eps_den, 1 <= eps_den < 2^31",
                (long long)eps_num, (long long)eps_den);
  return compile_common(mass, P, H, nqb, nkb, nkb_valid, 0, true, eps_num, eps_den, min_agree, row_ptr, col_idx,
                        nnz_cap, work_order, nnz_out, ws, ws_bytes, stream);
}

size_t calibatt_share_ws_bytes(int T, int H, int nqb, int nkb) {
  if (T < 1 || H < 1 || nqb < 1 || nkb < 1) return 0;
  const size_t rows = (size_t)H * nqb;
  const size_t W = ((size_t)nkb + 31) / 32;
  const size_t bits = (size_t)T * rows * W * 4;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  return 2 * up(bits) + up((size_t)T * rows * 4) + up(((size_t)T * rows + 1) * 4) + 256;
}

calibatt_status calibatt_share_timesteps(const int32_t* row_ptr, const int32_t* col_idx, const int64_t* set_off,
                                         int T, int H, int nqb, int nkb, int nkb_valid, double tau, double* iou,
                                         int32_t* cluster_of, int32_t* shared_row_ptr, int64_t* shared_set_off,
                                         int32_t* shared_col_idx, int64_t nnz_cap, int32_t* n_clusters_out,
                                         int64_t* nnz_out, void* ws, size_t ws_bytes, void* stream) {
  if (!row_ptr || !col_idx || !set_off || !iou || !cluster_of || !shared_row_ptr || !shared_set_off ||
      !n_clusters_out || !nnz_out || !ws)
    return fail(CALIBATT_ERR_NULL, "every pointer except shared_col_idx must be non-NULL");
  if (T < 1 || H < 1 || nqb < 1 || nkb < 1) return fail(CALIBATT_ERR_SHAPE, "T, H, nqb and nkb must be >= 1");
  if (T > 1024) return fail(CALIBATT_ERR_UNSUPPORTED, "T=%d exceeds 1024", T);
  if (nkb > calibatt::kMaxKeyBlocks) return fail(CALIBATT_ERR_UNSUPPORTED, "nkb=%d exceeds %d", nkb, calibatt::kMaxKeyBlocks);
  if (nkb_valid < 0 || nkb_valid > nkb) return fail(CALIBATT_ERR_SHAPE, "nkb_valid=%d must be in [0, nkb=%d]", nkb_valid, nkb);
  if (!(tau == tau)) return fail(CALIBATT_ERR_SHAPE, "tau must not be NaN");
  if (nnz_cap < 0) return fail(CALIBATT_ERR_SHAPE, "nnz_cap must be >= 0");
  if (nnz_cap > 0 && !shared_col_idx) return fail(CALIBATT_ERR_NULL, "shared_col_idx must be non-NULL when nnz_cap > 0");
  const long long rows = (long long)H * nqb;
  if ((long long)T * rows * nkb >= (1LL << 31)) return fail(CALIBATT_ERR_SHAPE, "T*H*nqb*nkb must be < 2^31");
  const size_t need = calibatt_share_ws_bytes(T, H, nqb, nkb);
  if (ws_bytes < need) return fail(CALIBATT_ERR_CAPACITY, "ws_bytes=%zu < %zu required", ws_bytes, need);
  if (!aligned(ws, 256) || !aligned(row_ptr, 4) || !aligned(col_idx, 4) || !aligned(set_off, 8) || !aligned(iou, 8) ||
      !aligned(cluster_of, 4) || !aligned(shared_row_ptr, 4) || !aligned(shared_set_off, 8) ||
      (shared_col_idx && !aligned(shared_col_idx, 4)))
    return fail(CALIBATT_ERR_ALIGN, "ws must be 256-byte aligned; int64/double arrays 8-, int32 arrays 4-byte aligned");

  calibatt::ShareArgs a;
  a.row_ptr = row_ptr;
  a.col_idx = col_idx;
  a.set_off = set_off;
  a.T = T;
  a.H = H;
  a.nqb = nqb;
  a.nkb = nkb;
  a.nkb_valid = nkb_valid;
  a.W = (nkb + 31) / 32;
  a.tau = tau;
  a.iou = iou;
  a.cluster_of = cluster_of;
  a.shared_row_ptr = shared_row_ptr;
  a.shared_set_off = shared_set_off;
  a.shared_col_idx = shared_col_idx;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  uint8_t* p = static_cast<uint8_t*>(ws);
  const size_t bits = (size_t)T * rows * a.W * 4;
  a.bits = reinterpret_cast<uint32_t*>(p);
  p += up(bits);
  a.shared_bits = reinterpret_cast<uint32_t*>(p);
  p += up(bits);
  a.counts = reinterpret_cast<int32_t*>(p);
  p += up((size_t)T * rows * 4);
  a.global_ptr = reinterpret_cast<int32_t*>(p);
  p += up(((size_t)T * rows + 1) * 4);
  a.n_clusters = reinterpret_cast<int32_t*>(p);

  hipStream_t st = (hipStream_t)stream;
  hipError_t e = calibatt::launch_share_cluster(a, st);
  if (e != hipSuccess) return hip_fail(e, "launching timestep clustering");
  int32_t C = 0;
  e = hipMemcpyAsync(&C, a.n_clusters, sizeof(int32_t), hipMemcpyDeviceToHost, st);
  if (e != hipSuccess) return hip_fail(e, "reading the cluster count");
  e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e, "synchronising after timestep clustering");
  if (C < 1 || C > T) return fail(CALIBATT_ERR_HIP, "cluster count %d out of range", C);
  *n_clusters_out = C;
  e = calibatt::launch_share_count(a, C, st);
  if (e != hipSuccess) return hip_fail(e, "launching shared-mask counts");
  int32_t total = 0;
  e = hipMemcpyAsync(&total, a.global_ptr + (size_t)C * rows, sizeof(int32_t), hipMemcpyDeviceToHost, st);
  if (e != hipSuccess) return hip_fail(e, "reading the shared kept count");
  e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e, "synchronising after shared-mask counts");
  *nnz_out = total;
  if (total > nnz_cap)
    return fail(CALIBATT_ERR_CAPACITY, "shared kept blocks %d exceed nnz_cap=%lld", total, (long long)nnz_cap);
  e = calibatt::launch_share_fill(a, C, st);
  if (e != hipSuccess) return hip_fail(e, "launching shared-mask fill");
  return ok();
}

size_t calibatt_skip_ws_bytes(int T, int H, int nqb) {
  if (T < 1 || H < 1 || nqb < 1) return 0;
  const size_t E = (size_t)T * H * nqb;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  return up(E * 4) + up((E + 1) * 4) + up((size_t)(calibatt::kMaxKeyBlocks / 2 + 1) * 4) + 256;
}

calibatt_status calibatt_encode_skip_lists(const int32_t* row_ptr, const int32_t* col_idx, const int64_t* set_off,
                                           int T, int H, int nqb, int nkb, int64_t merge_num, int64_t merge_den,
                                           int32_t* counts, int32_t* pairs, int width_cap, int32_t* width_out,
                                           int32_t* widest_out, void* ws, size_t ws_bytes, void* stream) {
  if (!row_ptr || !col_idx || !set_off || !counts || !width_out || !widest_out || !ws)
    return fail(CALIBATT_ERR_NULL, "every pointer except pairs must be non-NULL");
  if (T < 1 || H < 1 || nqb < 1 || nkb < 1) return fail(CALIBATT_ERR_SHAPE, "T, H, nqb and nkb must be >= 1");
  if (nkb > calibatt::kMaxKeyBlocks) return fail(CALIBATT_ERR_UNSUPPORTED, "nkb=%d exceeds %d", nkb, calibatt::kMaxKeyBlocks);
  if (merge_den < 1 || merge_num < 1 || merge_num > 100 * merge_den || merge_den > 2147483647LL)
    return fail(CALIBATT_ERR_SHAPE, "merge percentile %lld/%lld must lie in (0, 100]", (long long)merge_num,
                (long long)merge_den);
  if (width_cap < 0) return fail(CALIBATT_ERR_SHAPE, "width_cap must be >= 0");
  if (width_cap > 0 && !pairs) return fail(CALIBATT_ERR_NULL, "pairs must be non-NULL when width_cap > 0");
  const long long E = (long long)T * H * nqb;
  if (E * (long long)(nkb / 2 + 1) * 2 >= (1LL << 31)) return fail(CALIBATT_ERR_SHAPE, "T*H*nqb*(nkb/2+1)*2 must be < 2^31");
  const size_t need = calibatt_skip_ws_bytes(T, H, nqb);
  if (ws_bytes < need) return fail(CALIBATT_ERR_CAPACITY, "ws_bytes=%zu < %zu required", ws_bytes, need);
  if (!aligned(ws, 256) || !aligned(row_ptr, 4) || !aligned(col_idx, 4) || !aligned(set_off, 8) ||
      !aligned(counts, 4) || (pairs && !aligned(pairs, 4)))
    return fail(CALIBATT_ERR_ALIGN, "ws must be 256-byte aligned, set_off 8-byte, int32 arrays 4-byte aligned");
  calibatt::SkipArgs a;
  a.row_ptr = row_ptr;
  a.col_idx = col_idx;
  a.set_off = set_off;
  a.T = T;
  a.H = H;
  a.nqb = nqb;
  a.pct_num = merge_num;
  a.pct_den = merge_den;
  a.counts = counts;
  a.pairs = pairs;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  uint8_t* p = static_cast<uint8_t*>(ws);
  a.widths = reinterpret_cast<int32_t*>(p);
  p += up((size_t)E * 4) + up(((size_t)E + 1) * 4);
  a.hist = reinterpret_cast<int32_t*>(p);
  p += up((size_t)(calibatt::kMaxKeyBlocks / 2 + 1) * 4);
  a.width_dev = reinterpret_cast<int32_t*>(p);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = calibatt::launch_skip_widths(a, st);
  if (e != hipSuccess) return hip_fail(e, "launching skip-list widths");
  int32_t wd[2] = {0, 0};
  e = hipMemcpyAsync(wd, a.width_dev, sizeof(wd), hipMemcpyDeviceToHost, st);
  if (e != hipSuccess) return hip_fail(e, "reading the layer width");
  e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e, "synchronising after skip-list widths");
  *width_out = wd[0];
  *widest_out = wd[1];
  if (wd[0] > width_cap)
    return fail(CALIBATT_ERR_CAPACITY, "layer width %d exceeds width_cap=%d", wd[0], width_cap);
  e = calibatt::launch_skip_encode(a, st);
  if (e != hipSuccess) return hip_fail(e, "launching skip-list encode");
  return ok();
}

calibatt_status calibatt_decode_skip_lists(const int32_t* counts, const int32_t* pairs, int width, int T, int H,
                                           int nqb, int32_t* row_ptr, int64_t* set_off, int32_t* col_idx,
                                           int64_t nnz_cap, int64_t* nnz_out, void* ws, size_t ws_bytes,
                                           void* stream) {
  if (!counts || !row_ptr || !set_off || !nnz_out || !ws) return fail(CALIBATT_ERR_NULL, "counts, row_ptr, set_off, nnz_out and ws must be non-NULL");
  if (width > 0 && !pairs) return fail(CALIBATT_ERR_NULL, "pairs must be non-NULL when width > 0");
  if (T < 1 || H < 1 || nqb < 1 || width < 0) return fail(CALIBATT_ERR_SHAPE, "T, H, nqb must be >= 1 and width >= 0");
  if (width > calibatt::kMaxKeyBlocks / 2) return fail(CALIBATT_ERR_UNSUPPORTED, "width=%d exceeds %d", width, calibatt::kMaxKeyBlocks / 2);
  if (nnz_cap < 0) return fail(CALIBATT_ERR_SHAPE, "nnz_cap must be >= 0");
  if (nnz_cap > 0 && !col_idx) return fail(CALIBATT_ERR_NULL, "col_idx must be non-NULL when nnz_cap > 0");
  const long long E = (long long)T * H * nqb;
  if (E * (long long)calibatt::kMaxKeyBlocks >= (1LL << 31)) return fail(CALIBATT_ERR_SHAPE, "T*H*nqb*1024 must be < 2^31");
  const size_t need = calibatt_skip_ws_bytes(T, H, nqb);
  if (ws_bytes < need) return fail(CALIBATT_ERR_CAPACITY, "ws_bytes=%zu < %zu required", ws_bytes, need);
  if (!aligned(ws, 256) || !aligned(counts, 4) || (pairs && !aligned(pairs, 4)) || !aligned(row_ptr, 4) ||
      !aligned(set_off, 8) || (col_idx && !aligned(col_idx, 4)))
    return fail(CALIBATT_ERR_ALIGN, "ws must be 256-byte aligned, set_off 8-byte, int32 arrays 4-byte aligned");
  calibatt::SkipDecodeArgs a;
  a.counts = counts;
  a.pairs = pairs;
  a.W = width;
  a.T = T;
  a.H = H;
  a.nqb = nqb;
  a.row_ptr = row_ptr;
  a.set_off = set_off;
  a.col_idx = col_idx;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  uint8_t* p = static_cast<uint8_t*>(ws);
  a.kept = reinterpret_cast<int32_t*>(p);
  a.global_ptr = reinterpret_cast<int32_t*>(p + up((size_t)E * 4));
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = calibatt::launch_skip_decode_count(a, st);
  if (e != hipSuccess) return hip_fail(e, "launching skip-list decode (count)");
  int32_t total = 0;
  e = hipMemcpyAsync(&total, a.global_ptr + E, sizeof(int32_t), hipMemcpyDeviceToHost, st);
  if (e != hipSuccess) return hip_fail(e, "reading the decoded count");
  e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e, "synchronising after skip-list decode (count)");
  *nnz_out = total;
  if (total > nnz_cap) return fail(CALIBATT_ERR_CAPACITY, "decoded blocks %d exceed nnz_cap=%lld", total, (long long)nnz_cap);
  e = calibatt::launch_skip_decode_fill(a, st);
  if (e != hipSuccess) return hip_fail(e, "launching skip-list decode (fill)");
  return ok();
}

calibatt_status calibatt_build_schedule(const int32_t* row_ptr, int H, int nqb, int32_t* work_order,
                                        void* stream) {
  if (!row_ptr || !work_order) return fail(CALIBATT_ERR_NULL, "row_ptr and work_order must be non-NULL");
  if (H < 1 || nqb < 1) return fail(CALIBATT_ERR_SHAPE, "H and nqb must be >= 1");
  if (nqb > calibatt::kMaxKeyBlocks) return fail(CALIBATT_ERR_UNSUPPORTED, "nqb=%d exceeds %d", nqb, calibatt::kMaxKeyBlocks);
  if (H > calibatt::kMaxHeads) return fail(CALIBATT_ERR_UNSUPPORTED, "H=%d exceeds %d", H, calibatt::kMaxHeads);
  if (!aligned(row_ptr, 4) || !aligned(work_order, 4)) return fail(CALIBATT_ERR_ALIGN, "row_ptr and work_order must be 4-byte aligned");
  hipError_t e = calibatt::launch_schedule(row_ptr, H, nqb, work_order, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "launching work-order build");
  return ok();
}

size_t calibatt_similarity_ws_bytes(int B, int H, int L) {
  if (B < 1 || H < 1 || L < 128 || L % 128 != 0) return 0;
  const size_t bh = (size_t)B * H;
  return (bh * L * sizeof(float) + 255) / 256 * 256 + bh * (L / 128) * sizeof(double);
}

static calibatt_status check_grid(int frames, int grid_rows, int grid_cols, int seq_len) {
  if (frames < 1 || grid_rows < 1 || grid_cols < 1)
    return fail(CALIBATT_ERR_SHAPE, "frames=%d, grid_rows=%d and grid_cols=%d must be >= 1", frames, grid_rows, grid_cols);
  if ((long long)frames * grid_rows * grid_cols != seq_len)
    return fail(CALIBATT_ERR_SHAPE, "frames*grid_rows*grid_cols=%lld must equal seq_len=%d",
                (long long)frames * grid_rows * grid_cols, seq_len);
  return CALIBATT_OK;
}

calibatt_status calibatt_spatial_similarity(const void* Q, const void* K, int B, int H, int L, int seq_len,
                                            int d, calibatt_dtype dt, float scale, int frames, int grid_rows,
                                            int grid_cols, const float* lse_in, double* sim, void* ws,
                                            size_t ws_bytes, void* stream) {
  if (!Q || !K || !sim || !ws) return fail(CALIBATT_ERR_NULL, "Q, K, sim and ws must be non-NULL");
  if (!aligned(Q, 16) || !aligned(K, 16)) return fail(CALIBATT_ERR_ALIGN, "Q and K must be 16-byte aligned");
  if (!aligned(sim, 8) || !aligned(ws, 256)) return fail(CALIBATT_ERR_ALIGN, "sim must be 8-byte and ws 256-byte aligned");
  if (lse_in && !aligned(lse_in, 4)) return fail(CALIBATT_ERR_ALIGN, "lse_in must be 4-byte aligned");
  calibatt_status s = check_qkv_shape(B, H, L, seq_len, d, dt, 128);
  if (s != CALIBATT_OK) return s;
  if (dt != CALIBATT_BF16) return fail(CALIBATT_ERR_UNSUPPORTED, "spatial similarity supports bf16 inputs only");
  s = check_scale(scale);
  if (s != CALIBATT_OK) return s;
  s = check_grid(frames, grid_rows, grid_cols, seq_len);
  if (s != CALIBATT_OK) return s;
  if (grid_rows < 2) return fail(CALIBATT_ERR_SHAPE, "grid_rows=%d: the score needs at least two rows", grid_rows);
  const size_t need = calibatt_similarity_ws_bytes(B, H, L);
  if (ws_bytes < need) return fail(CALIBATT_ERR_CAPACITY, "ws_bytes=%zu, need %zu", ws_bytes, need);
  calibatt::SimArgs a;
  a.Q = Q;
  a.K = K;
  a.lse_in = lse_in;
  a.lse = static_cast<float*>(ws);
  a.part = reinterpret_cast<double*>(static_cast<char*>(ws) + ((size_t)B * H * L * sizeof(float) + 255) / 256 * 256);
  a.sim = sim;
  a.B = B;
  a.H = H;
  a.L = L;
  a.seq_len = seq_len;
  a.d = d;
  a.frames = frames;
  a.rows = grid_rows;
  a.cols = grid_cols;
  a.scale = scale;
  hipError_t e = calibatt::launch_spatial_similarity(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "launching spatial similarity");
  return ok();
}

calibatt_status calibatt_select_repetitive_heads(const double* sim, int P, int H, double tau, int32_t* heads,
                                                 int32_t* n_heads, void* stream) {
  if (!sim || !heads || !n_heads) return fail(CALIBATT_ERR_NULL, "sim, heads and n_heads must be non-NULL");
  if (P < 1 || H < 1) return fail(CALIBATT_ERR_SHAPE, "P=%d and H=%d must be >= 1", P, H);
  if (!aligned(sim, 8)) return fail(CALIBATT_ERR_ALIGN, "sim must be 8-byte aligned");
  std::vector<double> host((size_t)P * H);
  hipError_t e = hipMemcpyAsync(host.data(), sim, host.size() * sizeof(double), hipMemcpyDeviceToHost,
                                (hipStream_t)stream);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "reading the similarity scores");
  int n = 0;
  for (int h = 0; h < H; ++h) {
    double acc = 0.0;
    for (int p = 0; p < P; ++p) acc += host[(size_t)p * H + h];
    if (acc / P > tau) heads[n++] = h;
  }
  *n_heads = n;
  return ok();
}

static long long anchor_queries(int frames, int grid_cols, int k_anchor) {
  return (long long)frames * k_anchor * grid_cols;
}

size_t calibatt_anchor_ws_bytes(int B, int H, int frames, int grid_cols, int k_anchor, int d) {
  if (B < 1 || H < 1 || frames < 1 || grid_cols < 1 || k_anchor < 1 || (d != 64 && d != 128)) return 0;
  const long long Lq = (anchor_queries(frames, grid_cols, k_anchor) + 127) / 128 * 128;
  const size_t oa = ((size_t)B * H * Lq * d * 2 + 255) / 256 * 256;
  return oa + ((size_t)H * (Lq / 128) * calibatt::kMaxSplit + calibatt::kParts + 1) * sizeof(int32_t);
}

calibatt_status calibatt_anchor_attn_fwd(const void* Q, const void* K, const void* V, void* O,
                                         const int32_t* heads, int n_heads, int frames, int grid_rows,
                                         int grid_cols, int k_anchor, float scale, int B, int H, int L,
                                         int seq_len, int d, calibatt_dtype dt, int32_t* queue_ws,
                                         calibatt_vlayout v_layout, void* ws, size_t ws_bytes, void* stream) {
  calibatt_status s = check_ptrs4(Q, K, V, O);
  if (s != CALIBATT_OK) return s;
  s = check_qkv_shape(B, H, L, seq_len, d, dt, 128);
  if (s != CALIBATT_OK) return s;
  if (dt != CALIBATT_BF16) return fail(CALIBATT_ERR_UNSUPPORTED, "anchor attention supports bf16 inputs only");
  s = check_v_layout(v_layout);
  if (s != CALIBATT_OK) return s;
  s = check_scale(scale);
  if (s != CALIBATT_OK) return s;
  s = check_out_alias(Q, K, V, O, B, H, L, d, dt);
  if (s != CALIBATT_OK) return s;
  s = check_grid(frames, grid_rows, grid_cols, seq_len);
  if (s != CALIBATT_OK) return s;
  if (k_anchor < 1 || k_anchor > grid_rows)
    return fail(CALIBATT_ERR_SHAPE, "k_anchor=%d must be in [1, grid_rows=%d]", k_anchor, grid_rows);
  if (n_heads < 0 || n_heads > H) return fail(CALIBATT_ERR_SHAPE, "n_heads=%d must be in [0, H=%d]", n_heads, H);
  if (n_heads > calibatt::kMaxListHeads)
    return fail(CALIBATT_ERR_UNSUPPORTED, "n_heads=%d exceeds %d", n_heads, calibatt::kMaxListHeads);
  if (n_heads > 0 && !heads) return fail(CALIBATT_ERR_NULL, "heads must be non-NULL when n_heads > 0");
  if (!queue_ws || !ws) return fail(CALIBATT_ERR_NULL, "queue_ws and ws must be non-NULL");
  if (!aligned(queue_ws, 16) || !aligned(ws, 256)) return fail(CALIBATT_ERR_ALIGN, "queue_ws must be 16-byte and ws 256-byte aligned");
  calibatt::AnchorArgs a;
  a.heads.n = n_heads;
  for (int i = 0; i < n_heads; ++i) {
    if (heads[i] < 0 || heads[i] >= H) return fail(CALIBATT_ERR_SHAPE, "heads[%d]=%d outside [0, H=%d)", i, heads[i], H);
    for (int j = 0; j < i; ++j)
      if (heads[j] == heads[i]) return fail(CALIBATT_ERR_SHAPE, "head %d is listed twice", heads[i]);
    a.heads.h[i] = heads[i];
  }
  const long long La = anchor_queries(frames, grid_cols, k_anchor);
  const long long Lq = (La + 127) / 128 * 128;
  if ((long long)B * H * Lq * d >= (1LL << 31)) return fail(CALIBATT_ERR_SHAPE, "B*H*Lq*d must be < 2^31");
  const size_t need = calibatt_anchor_ws_bytes(B, H, frames, grid_cols, k_anchor, d);
  if (ws_bytes < need) return fail(CALIBATT_ERR_CAPACITY, "ws_bytes=%zu, need %zu", ws_bytes, need);
  if (n_heads == 0) return ok();
  int ncu = 256;
  hipError_t e = cu_count(&ncu);
  if (e != hipSuccess) return hip_fail(e, "querying the compute-unit count");
  const size_t oa = ((size_t)B * H * Lq * d * 2 + 255) / 256 * 256;
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.v_transposed = v_layout == CALIBATT_V_BHDL;
  a.O = O;
  a.Oa = ws;
  a.order = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + oa);
  a.queue = queue_ws;
  a.B = B;
  a.H = H;
  a.L = L;
  a.seq_len = seq_len;
  a.d = d;
  a.rows = grid_rows;
  a.cols = grid_cols;
  a.k = k_anchor;
  a.La = (int)La;
  a.Lq = (int)Lq;
  a.scale = scale;
  a.num_cu = ncu;
  e = calibatt::launch_anchor_fwd(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "launching anchor-row attention");
  return ok();
}

int calibatt_anchor_parts(int B, int n_heads, int frames, int grid_cols, int k_anchor, int L, int seq_len, int d,
                          int num_cu) {
  if (B < 1 || n_heads < 1 || frames < 1 || grid_cols < 1 || k_anchor < 1 || seq_len < 1 || L < seq_len ||
      (d != 64 && d != 128) || num_cu < 1)
    return 0;
  const long long Lq = (anchor_queries(frames, grid_cols, k_anchor) + 127) / 128 * 128;
  return 1 << calibatt::anchor_split_shift((long long)B * n_heads * (Lq / 128), 2 * num_cu, (seq_len + 127) / 128,
                                           Lq, L, d);
}

calibatt_status calibatt_validate_csr(const int32_t* row_ptr, const int32_t* col_idx, int rows,
                                      int nkb_valid, int64_t nnz) {
  if (!row_ptr) return fail(CALIBATT_ERR_NULL, "row_ptr must be non-NULL");
  if (rows < 0 || nkb_valid < 0 || nnz < 0) return fail(CALIBATT_ERR_SHAPE, "rows, nkb_valid and nnz must be >= 0");
  if (nnz > 0 && !col_idx) return fail(CALIBATT_ERR_NULL, "col_idx must be non-NULL when nnz > 0");
  if (row_ptr[0] != 0) return fail(CALIBATT_ERR_CSR, "row_ptr[0]=%d, expected 0", row_ptr[0]);
  for (int r = 0; r < rows; ++r) {
    const int32_t a = row_ptr[r], b = row_ptr[r + 1];
    if (b < a) return fail(CALIBATT_ERR_CSR, "row_ptr decreases at row %d (%d -> %d)", r, a, b);
    if (b > nnz) return fail(CALIBATT_ERR_CSR, "row_ptr[%d]=%d exceeds nnz=%lld", r + 1, b, (long long)nnz);
    for (int32_t i = a; i < b; ++i) {
      const int32_t kb = col_idx[i];
      if (kb < 0 || kb >= nkb_valid) return fail(CALIBATT_ERR_CSR, "row %d: column %d outside [0, %d)", r, kb, nkb_valid);
      if (i > a && kb <= col_idx[i - 1])
        return fail(CALIBATT_ERR_CSR, "row %d: columns not strictly ascending (%d after %d)", r, kb, col_idx[i - 1]);
    }
  }
  if (row_ptr[rows] != nnz) return fail(CALIBATT_ERR_CSR, "row_ptr[rows]=%d differs from nnz=%lld", row_ptr[rows], (long long)nnz);
  return ok();
}

const char* calibatt_status_string(calibatt_status s) {
  switch (s) {
    case CALIBATT_OK: return "ok";
    case CALIBATT_ERR_NULL: return "null pointer";
    case CALIBATT_ERR_SHAPE: return "bad shape";
    case CALIBATT_ERR_DTYPE: return "bad dtype";
    case CALIBATT_ERR_ALIGN: return "misaligned pointer";
    case CALIBATT_ERR_CSR: return "malformed kept-block list";
    case CALIBATT_ERR_CAPACITY: return "output buffer too small";
    case CALIBATT_ERR_UNSUPPORTED: return "unsupported combination";
    case CALIBATT_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* calibatt_last_error(void) { return g_last_error.c_str(); }

int calibatt_version(void) { return CALIBATT_VERSION; }

}  // extern "C"
