// lds_probes.hip -- the two measurements behind the ring kernel's LDS
// layouts (bench.py --lds-probes).  Output: one JSON object per line.
//
// 1. LDS read rate of one wave's fragment read in each candidate layout:
//    1024 workgroups of 4 waves, each wave issuing 16 reads per iteration
//    (all in one asm block, so the compiler neither merges nor reorders
//    them); TB/s from hip events, and the shader-clock cycles per read from
//    s_memtime.  The bank-conflict cycles of each pattern are read with
//    rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_INSTS_LDS over this program.
// 2. Direct-to-LDS load rate (buffer_load_dwordx4 ... lds, 1 KiB per
//    instruction) for the global footprints an operand tile can have: 16
//    rows x 64 bytes, 8 rows x 128 bytes (lanes in row order, or the two
//    64-byte halves of each row in the two halves of the wave), 2 rows x 512
//    bytes; rows 16 KiB apart, from a 32 MiB matrix (L2 and last-level cache)
//    and a 256 MiB one.
//
// Every LDS address stays inside the workgroup's 64 KiB array (checked on
// the host before any launch); global reads are bounded by the buffer
// resource.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#define CHECK(x)                                                                           \
    do {                                                                                   \
        hipError_t e_ = (x);                                                               \
        if (e_ != hipSuccess) {                                                            \
            fprintf(stderr, "lds_probes: %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            exit(1);                                                                       \
        }                                                                                  \
    } while (0)

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int LDS = 65536;
constexpr int ITERS = 512;

// ------------------------------------------------------------ read patterns
// Byte address of read j (0..15) of lane l.  A k-contiguous fragment read:
// lane l takes row 16 f + l % 16, chunk q = l / 16 (16 bytes = 8 k) of a
// tile with 64-byte rows (one step of 32 k); f = j % 8.
enum ReadPattern {
    R_CONTIG,        // ds_read_b128, lane l at 16 l (a contiguous KiB)
    R_ROWS_PLAIN,    // ds_read_b128, rows of 64 bytes, no swizzle
    R_ROWS_KEY_R4,   // ... chunk q ^ ((r / 4) % 4)
    R_ROWS_KEY_R,    // ... chunk q ^ (r % 4)
    R_ROWS_KEY_R2,   // ... chunk q ^ ((r / 2) % 4)        (the kernel, one-step stages)
    R_BLOCKS_KEY_R2, // ... two-step stages: 1 KiB blocks of 8 rows, each step's 64 bytes
                     //     of the 8 rows together; step j / 8   (the kernel, two-step stages)
    R_TR_KS,         // ds_read_b64_tr_b16 of a k-strided tile, 512-byte k-rows, the kernel's key
    R_COUNT
};
const char* kReadNames[R_COUNT] = {"ds_read_b128 contiguous KiB", "ds_read_b128 rows, no swizzle",
                                   "ds_read_b128 rows, key (r/4)%4", "ds_read_b128 rows, key r%4",
                                   "ds_read_b128 rows, key (r/2)%4", "ds_read_b128 two-step blocks, key (r/2)%4",
                                   "ds_read_b64_tr_b16 k-rows, key 4(r%4)^2((r/8)%2)"};

__host__ __device__ int read_addr(int P, int l, int j) {
    const int q = l >> 4, i = l & 15, f = j & 7, r = 16 * f + i;
    switch (P) {
        case R_CONTIG: return f * 1024 + 16 * l;
        case R_ROWS_PLAIN: return r * 64 + 16 * q;
        case R_ROWS_KEY_R4: return r * 64 + 16 * (q ^ ((r >> 2) & 3));
        case R_ROWS_KEY_R: return r * 64 + 16 * (q ^ (r & 3));
        case R_ROWS_KEY_R2: return r * 64 + 16 * (q ^ ((r >> 1) & 3));
        case R_BLOCKS_KEY_R2: return (r >> 3) * 1024 + (j >> 3) * 512 + (r & 7) * 64 + 16 * (q ^ ((r >> 1) & 3));
        case R_TR_KS: {
            // lane i of group q: k-row 8q + i/4 (+4 for odd j), 16 columns of fragment j/2
            const int kr = 8 * q + (i >> 2) + 4 * (j & 1);
            const int c = 2 * (j >> 1) + ((i & 3) >> 1);
            return kr * 512 + 16 * (c ^ (4 * (kr & 3) ^ 2 * ((kr >> 3) & 1))) + 8 * (i & 1);
        }
    }
    return 0;
}
__host__ __device__ int read_bytes(int P) { return P == R_TR_KS ? 8 : 16; }

#define READ16(INSTR)                                                                                               \
    asm volatile(INSTR " %0, %16\n\t" INSTR " %1, %17\n\t" INSTR " %2, %18\n\t" INSTR " %3, %19\n\t" INSTR          \
                       " %4, %20\n\t" INSTR " %5, %21\n\t" INSTR " %6, %22\n\t" INSTR " %7, %23\n\t" INSTR          \
                       " %8, %24\n\t" INSTR " %9, %25\n\t" INSTR " %10, %26\n\t" INSTR " %11, %27\n\t" INSTR        \
                       " %12, %28\n\t" INSTR " %13, %29\n\t" INSTR " %14, %30\n\t" INSTR " %15, %31\n\t"           \
                       "s_waitcnt lgkmcnt(0)"                                                                       \
                 : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]),      \
                   "=&v"(v[7]), "=&v"(v[8]), "=&v"(v[9]), "=&v"(v[10]), "=&v"(v[11]), "=&v"(v[12]), "=&v"(v[13]),   \
                   "=&v"(v[14]), "=&v"(v[15])                                                                       \
                 : "v"(b[0]), "v"(b[1]), "v"(b[2]), "v"(b[3]), "v"(b[4]), "v"(b[5]), "v"(b[6]), "v"(b[7]),          \
                   "v"(b[8]), "v"(b[9]), "v"(b[10]), "v"(b[11]), "v"(b[12]), "v"(b[13]), "v"(b[14]), "v"(b[15])     \
                 : "memory")

template <int P>
__global__ __launch_bounds__(256) void read_probe(uint32_t* out, unsigned long long* clk) {
    __shared__ __attribute__((aligned(1024))) char smem[LDS];
    for (int i = threadIdx.x; i < LDS / 4; i += 256) ((uint32_t*)smem)[i] = i;
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t base = (uint32_t)(uintptr_t)(lds_void*)smem + (wave & 1) * 16384;
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    uint32_t acc = 0;
    for (int it = 0; it < ITERS; ++it) {
        uint32_t b[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) b[j] = base + (it & 1) * 32768 + read_addr(P, lane, j);
        if constexpr (P == R_TR_KS) {
            u32x2 v[16];
            READ16("ds_read_b64_tr_b16");
#pragma unroll
            for (int j = 0; j < 16; ++j) acc ^= v[j][0] ^ v[j][1];
        } else {
            u32x4 v[16];
            READ16("ds_read_b128");
#pragma unroll
            for (int j = 0; j < 16; ++j) acc ^= v[j][0] ^ v[j][3];
        }
    }
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    out[blockIdx.x * 256 + threadIdx.x] = acc;
    if (threadIdx.x == 0) clk[blockIdx.x] = t1 - t0;
}

// ------------------------------------------------------------ load patterns
enum LoadPattern { L_ROWS64, L_ROWS128, L_ROWS128_HALVES, L_ROWS512, L_COUNT };
const char* kLoadNames[L_COUNT] = {"16 rows x 64 bytes", "8 rows x 128 bytes",
                                   "8 rows x 128 bytes, 64-byte halves in the two half-waves", "2 rows x 512 bytes"};
constexpr int PITCH = 16384;  // bytes between rows (8192 fp16)

template <int P>
__global__ __launch_bounds__(256) void load_probe(const char* buf, int64_t bytes, int rows_total, int iters, int* out) {
    __shared__ __attribute__((aligned(1024))) char smem[LDS];
    const int base = (int)(uintptr_t)(lds_void*)smem;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint64_t a = (uint64_t)buf;
    const uint32_t n = bytes > 0xffffffffLL ? 0xffffffffu : (uint32_t)bytes;
    const i32x4 rs = {__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                      __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32)), __builtin_amdgcn_readfirstlane((int)n),
                      0x00020000};
    constexpr int RPI = P == L_ROWS64 ? 16 : P == L_ROWS512 ? 2 : 8;  // rows per instruction
    constexpr int BPR = 1024 / RPI;                                   // bytes per row
    const int r_in = P == L_ROWS128_HALVES ? (lane % 32) / 4 : lane / (BPR / 16);
    const int c_in = P == L_ROWS128_HALVES ? (lane / 32) * 4 + lane % 4 : lane % (BPR / 16);
    const int panel = (int)(((int64_t)blockIdx.x * 256) % rows_total);  // 256 rows per workgroup
    int voff[4];
    for (int x = 0; x < 4; ++x) voff[x] = (panel + wave * 64 + x * 16 + r_in) * PITCH + c_in * 16;
    for (int it = 0; it < iters; ++it) {
        const int so = (it * BPR) % PITCH;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int m0 = base + ((it & 3) * 16 + wave * 4 + x) * 1024;
            asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                         :
                         : "s"(__builtin_amdgcn_readfirstlane(m0)), "v"(voff[x]), "s"(rs), "s"(so)
                         : "memory");
        }
        if ((it & 3) == 3) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    out[blockIdx.x * 256 + threadIdx.x] = ((int*)smem)[threadIdx.x];
}

template <int P>
void run_read(uint32_t* d_out, unsigned long long* d_clk, int blocks, hipEvent_t e0, hipEvent_t e1) {
    read_probe<P><<<blocks, 256>>>(d_out, d_clk);
    CHECK(hipGetLastError());
    CHECK(hipDeviceSynchronize());
    CHECK(hipEventRecord(e0));
    read_probe<P><<<blocks, 256>>>(d_out, d_clk);
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    unsigned long long* h = (unsigned long long*)malloc(sizeof(unsigned long long) * blocks);
    CHECK(hipMemcpy(h, d_clk, sizeof(unsigned long long) * blocks, hipMemcpyDeviceToHost));
    double cyc = 0;
    for (int i = 0; i < blocks; ++i) cyc += (double)h[i];
    cyc /= blocks;
    free(h);
    const double reads_per_wave = (double)ITERS * 16;
    const double bytes = (double)blocks * 256 * reads_per_wave * read_bytes(P);
    printf("{\"probe\": \"lds_read\", \"pattern\": \"%s\", \"ms\": %.4f, \"TB_s\": %.2f, "
           "\"memtime_cycles_per_read_per_wave\": %.2f}\n",
           kReadNames[P], ms, bytes / (ms * 1e-3) / 1e12, cyc / reads_per_wave);
    fflush(stdout);
}

template <int P>
void run_load(const char* buf, int rows, int* d_out, int blocks, hipEvent_t e0, hipEvent_t e1) {
    const int iters = 256;
    const int64_t bytes = (int64_t)rows * PITCH;
    load_probe<P><<<blocks, 256>>>(buf, bytes, rows, iters, d_out);
    CHECK(hipGetLastError());
    CHECK(hipDeviceSynchronize());
    CHECK(hipEventRecord(e0));
    for (int r = 0; r < 3; ++r) load_probe<P><<<blocks, 256>>>(buf, bytes, rows, iters, d_out);
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    ms /= 3;
    const double b = (double)blocks * 16 * iters * 1024;
    printf("{\"probe\": \"lds_load\", \"pattern\": \"%s\", \"matrix_MiB\": %d, \"ms\": %.4f, \"TB_s\": %.2f}\n",
           kLoadNames[P], (int)(bytes >> 20), ms, b / (ms * 1e-3) / 1e12);
    fflush(stdout);
}

}  // namespace

int main() {
    // every LDS address of every read pattern inside the array
    for (int P = 0; P < R_COUNT; ++P)
        for (int l = 0; l < 64; ++l)
            for (int j = 0; j < 16; ++j) {
                const int a = read_addr(P, l, j);
                if (a < 0 || a % read_bytes(P) != 0 || a + read_bytes(P) + 16384 + 32768 > LDS) {
                    fprintf(stderr, "lds_probes: read pattern %d leaves the LDS array\n", P);
                    return 1;
                }
            }
    // every load writes LDS blocks 0..63 and reads rows panel .. panel + 255
    const int blocks = 1024;
    uint32_t* d_out;
    unsigned long long* d_clk;
    CHECK(hipMalloc(&d_out, blocks * 256 * sizeof(uint32_t)));
    CHECK(hipMalloc(&d_clk, blocks * sizeof(unsigned long long)));
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    run_read<R_CONTIG>(d_out, d_clk, blocks, e0, e1);
    run_read<R_ROWS_PLAIN>(d_out, d_clk, blocks, e0, e1);
    run_read<R_ROWS_KEY_R4>(d_out, d_clk, blocks, e0, e1);
    run_read<R_ROWS_KEY_R>(d_out, d_clk, blocks, e0, e1);
    run_read<R_ROWS_KEY_R2>(d_out, d_clk, blocks, e0, e1);
    run_read<R_BLOCKS_KEY_R2>(d_out, d_clk, blocks, e0, e1);
    run_read<R_TR_KS>(d_out, d_clk, blocks, e0, e1);

    const int rows_max = 16384;  // 256 MiB
    char* buf;
    CHECK(hipMalloc(&buf, (size_t)rows_max * PITCH));
    CHECK(hipMemset(buf, 1, (size_t)rows_max * PITCH));
    int* d_lout;
    CHECK(hipMalloc(&d_lout, 2048 * 256 * sizeof(int)));
    for (int rows : {2048, rows_max}) {
        run_load<L_ROWS64>(buf, rows, d_lout, 2048, e0, e1);
        run_load<L_ROWS128>(buf, rows, d_lout, 2048, e0, e1);
        run_load<L_ROWS128_HALVES>(buf, rows, d_lout, 2048, e0, e1);
        run_load<L_ROWS512>(buf, rows, d_lout, 2048, e0, e1);
    }
    return 0;
}
