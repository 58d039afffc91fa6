/* Test-only stand-ins for two HIP runtime entry points, preloaded into a
 * host-only test process so that ttt_la_create reaches its allocation on a
 * machine without a GPU and sees it fail:
 *   hipGetDevice  reports device 0;
 *   hipMalloc     fails with the status in ALLOC_FAIL_STATUS (default 2,
 *                 hipErrorOutOfMemory) and counts its calls.
 * Everything else resolves to the real runtime. */
#include <stddef.h>
#include <stdlib.h>

static int n_malloc_calls = 0;

int hipGetDevice(int* device) {
    if (device) *device = 0;
    return 0;
}

int hipMalloc(void** ptr, size_t size) {
    (void)size;
    ++n_malloc_calls;
    if (ptr) *ptr = NULL;
    const char* s = getenv("ALLOC_FAIL_STATUS");
    return s ? atoi(s) : 2;
}

int alloc_fail_shim_calls(void) { return n_malloc_calls; }
