"""Reference block allocator with reference counts (oracle; test infrastructure).

Follows "KV cache and PagedAttention" (askaiml.pages.dev), §4 "PagedAttention":
pages are all the same size, so any free page serves any request and one
allocation or release is a constant-time operation; requests with a common
prefix may map the same physical pages.  The "KV Cache" glossary
(inferensys.com, PagedAttention block management) adds that blocks are shared
across sequences for parallel sampling and beam search.

The pages fix neither the order in which free pages are handed out nor how
sharing is tracked.  Readings taken here (the library must return the same ids
bit for bit):

* Free pages form a LIFO stack.  It starts from `initial_free_order`; the first
  allocation returns initial_free_order[0], the next one initial_free_order[1],
  and so on.  A page whose count drops to zero is pushed on top, so it is the
  next one handed out.
* Each page carries a reference count: allocation sets it to 1, `retain` adds
  one mapping, `release` drops one and returns the page to the stack at zero.
* Retaining or releasing a page that is out of range or not allocated is an
  error (BadBlock); allocating from an empty stack is an error (NoBlocks).
  State is left unchanged by a failed call.
"""


class AllocError(Exception):
    """Base class of allocator errors."""


class NoBlocks(AllocError):
    """No free page is left."""


class BadBlock(AllocError):
    """Page id out of range, or not currently allocated."""


class RefAllocator:
    def __init__(self, num_blocks, initial_free_order=None):
        if num_blocks <= 0:
            raise ValueError("num_blocks must be positive")
        order = list(range(num_blocks)) if initial_free_order is None \
            else [int(x) for x in initial_free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("initial_free_order must be a permutation of 0..N-1")
        self.num_blocks = num_blocks
        # top of the stack is the end of the list
        self._stack = list(reversed(order))
        self._rc = [0] * num_blocks

    def alloc(self):
        if not self._stack:
            raise NoBlocks()
        b = self._stack.pop()
        self._rc[b] = 1
        return b

    def _check_live(self, b):
        if not (0 <= b < self.num_blocks) or self._rc[b] == 0:
            raise BadBlock(b)

    def retain(self, b):
        self._check_live(b)
        self._rc[b] += 1

    def release(self, b):
        self._check_live(b)
        self._rc[b] -= 1
        if self._rc[b] == 0:
            self._stack.append(b)

    def refcount(self, b):
        if not (0 <= b < self.num_blocks):
            raise BadBlock(b)
        return self._rc[b]

    def num_free(self):
        return len(self._stack)

    def free_list_top_first(self):
        """Free pages in the order the next allocations would return them."""
        return list(reversed(self._stack))
