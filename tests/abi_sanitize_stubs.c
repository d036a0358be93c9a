/*
 * abi_sanitize_stubs.c -- a stand-in for the few HIP runtime entry points
 * that the host side of libpsq calls, so that the library's host code (the
 * C ABI's validation, workspace sizing, copy planning and launch set-up)
 * can run on a CPU under AddressSanitizer and UndefinedBehaviorSanitizer.
 * Nothing here touches a GPU: a "launch" checks the launch shape against
 * HIP's limits, counts it and returns success.  Test infrastructure only.
 */
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

typedef struct {
    uint32_t x, y, z;
} stub_dim3;
typedef int stub_error;   /* hipSuccess == 0 */

long stub_launches;
static stub_dim3 pushed_grid, pushed_block;
static size_t pushed_shared;
static void *pushed_stream;
static char fake_module[64];
static char fake_symbol_memory[256];

/* every launch: a 1-D grid of at least one workgroup, at most 1024 threads
 * per workgroup, and fewer than 2^32 threads in all */
static void check_shape(stub_dim3 grid, stub_dim3 block)
{
    const uint64_t threads = (uint64_t)grid.x * grid.y * grid.z * block.x * block.y * block.z;
    if (grid.x < 1 || grid.y != 1 || grid.z != 1 || block.x < 1 || block.x > 1024 ||
        block.y != 1 || block.z != 1 || threads > 0xffffffffull) {
        fprintf(stderr, "bad launch shape: grid %u,%u,%u block %u,%u,%u\n", grid.x, grid.y,
                grid.z, block.x, block.y, block.z);
        abort();
    }
}

void **__hipRegisterFatBinary(const void *data)
{
    (void)data;
    return (void **)fake_module;
}

void __hipUnregisterFatBinary(void **module) { (void)module; }

void __hipRegisterFunction(void **module, const void *host_fn, char *device_fn,
                           const char *device_name, unsigned int thread_limit, void *tid,
                           void *bid, void *block_dim, void *grid_dim, int *wsize)
{
    (void)module; (void)host_fn; (void)device_fn; (void)device_name; (void)thread_limit;
    (void)tid; (void)bid; (void)block_dim; (void)grid_dim; (void)wsize;
}

void __hipRegisterVar(void **module, void *var, char *host_var, char *device_var, int ext,
                      size_t size, int constant, int global)
{
    (void)module; (void)var; (void)host_var; (void)device_var; (void)ext; (void)size;
    (void)constant; (void)global;
}

stub_error __hipPushCallConfiguration(stub_dim3 grid, stub_dim3 block, size_t shared,
                                      void *stream)
{
    pushed_grid = grid;
    pushed_block = block;
    pushed_shared = shared;
    pushed_stream = stream;
    return 0;
}

stub_error __hipPopCallConfiguration(stub_dim3 *grid, stub_dim3 *block, size_t *shared,
                                     void **stream)
{
    *grid = pushed_grid;
    *block = pushed_block;
    *shared = pushed_shared;
    *stream = pushed_stream;
    return 0;
}

stub_error hipLaunchKernel(const void *fn, stub_dim3 grid, stub_dim3 block, void **args,
                           size_t shared, void *stream)
{
    (void)fn; (void)args; (void)shared; (void)stream;
    check_shape(grid, block);
    ++stub_launches;
    return 0;
}

stub_error hipGetLastError(void) { return 0; }

stub_error hipGetDevice(int *device)
{
    *device = 0;
    return 0;
}

stub_error hipGetSymbolAddress(void **ptr, const void *symbol)
{
    (void)symbol;
    *ptr = fake_symbol_memory;
    return 0;
}
