# empty
